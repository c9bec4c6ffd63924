// Device-side building blocks shared by every generated class kernel.
//
// Source: "FusionRCG: Orchestrating Recursive Computation Graphs across GPU
// Memory Hierarchies".  Section II-A: the recurrence starts from Boys values
// F_m(T) and the Gaussian-product quantities zeta, eta, rho, P, Q, W of Eq. (2);
// Algorithm 2 (section III-C) forms them per primitive quartet
// (its Gaussian-pair and Boys steps) inside the primitive loops.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// ---------------------------------------------------------------------------
// Boys function table: rows T_k = k / ERI_BT_PER_UNIT for T_k in [0, ERI_BT_TMAX];
// row k holds exp(-T_k) followed by F_0(T_k) .. F_{ERI_BT_MMAX}(T_k).
// ---------------------------------------------------------------------------
#define ERI_BT_PER_UNIT 32
#define ERI_BT_TMAX 36
#define ERI_BT_ROWS (ERI_BT_TMAX * ERI_BT_PER_UNIT + 1)
#define ERI_BT_MMAX 22
#define ERI_BT_COLS (ERI_BT_MMAX + 2)
#define ERI_LMAX 4
#define ERI_PP_STRIDE 10
// memory-tier grid: at most this many workgroups, each owning one scratch slice
#define ERI_MEM_WGS 1024

struct EriPrimPair {
    double zeta;   // alpha + beta
    double izeta;  // 1 / zeta
    double P[3];   // (alpha A + beta B) / zeta
    double PA[3];  // P - A
    double Kc;     // c_a c_b exp(-alpha beta |AB|^2 / zeta) / zeta
};

struct EriQuartetGeom {
    double WP[3], WQ[3];
    double T, pref, roz, roe, i2ze;
};

struct EriClassArgs {
    const int* qbra;        // [nq] bra pair of each quartet
    const int* qket;        // [nq] ket pair of each quartet
    int nq;
    const int4* pair_info;  // per pair: shell a, shell b, first primitive pair, primitive pairs
    const double* ppd;      // primitive-pair records, ERI_PP_STRIDE doubles each
    const double* cen;      // shell centres [3 * nshell]
    const double* boys;     // Boys table [ERI_BT_ROWS * ERI_BT_COLS]
    double* out;            // quartet q writes out[q * block_size ...]
    double* scratch;        // memory-tier scratch (scratch_wgs workgroup slices)
    int scratch_wgs;
    int grid_cap;           // register tier: persistent grid size (workgroups)
    long long pair_base;    // >= 0: qbra[q] = pair_base + 2q and qket[q] = qbra[q] + 1 (explicit lists)
};

typedef void (*EriLaunchFn)(const EriClassArgs&, hipStream_t);

struct EriClassEntry {
    int class_id;
    int spherical;
    int la, lb, lc, ld;
    char tier;                 // 'V' register tier, 'M' memory tier
    long long scratch_doubles; // per workgroup, memory tier only
    EriLaunchFn launch;        // any contraction degree
    EriLaunchFn launch_k1;     // every quartet uncontracted (K_a K_b K_c K_d = 1)
};

extern EriClassEntry eri_class_table[];  // host-only (non-const keeps it out of device code)
extern const int eri_class_table_size;

__device__ __forceinline__ EriPrimPair eri_load_pp(const double* __restrict__ ppd, int idx)
{
    const double2* p = reinterpret_cast<const double2*>(ppd + (size_t)idx * ERI_PP_STRIDE);
    const double2 v0 = p[0], v1 = p[1], v2 = p[2], v3 = p[3], v4 = p[4];
    EriPrimPair r;
    r.zeta = v0.x;
    r.izeta = v0.y;
    r.P[0] = v1.x;
    r.P[1] = v1.y;
    r.P[2] = v2.x;
    r.PA[0] = v2.y;
    r.PA[1] = v3.x;
    r.PA[2] = v3.y;
    r.Kc = v4.x;
    return r;
}

// Gaussian-product quantities of one primitive quartet.  For the ket pair the
// record's PA field holds Q - C.  W = (zeta P + eta Q)/(zeta + eta), so
// W - P = eta (Q - P)/(zeta+eta) and W - Q = zeta (P - Q)/(zeta+eta).  P - Q is
// formed as (P - A) - (Q - C) + (A - C) from coordinate differences, so it is
// exactly zero when all four centres coincide.
__device__ __forceinline__ void eri_geom(const EriPrimPair& B, const EriPrimPair& K, double ACx, double ACy,
                                         double ACz, EriQuartetGeom& g)
{
    const double ze = B.zeta + K.zeta;
    const double ize = 1.0 / ze;
    const double PQx = (B.PA[0] - K.PA[0]) + ACx, PQy = (B.PA[1] - K.PA[1]) + ACy, PQz = (B.PA[2] - K.PA[2]) + ACz;
    const double rho = B.zeta * K.zeta * ize;
    const double ke = K.zeta * ize, kz = B.zeta * ize;
    g.WP[0] = -ke * PQx;
    g.WP[1] = -ke * PQy;
    g.WP[2] = -ke * PQz;
    g.WQ[0] = kz * PQx;
    g.WQ[1] = kz * PQy;
    g.WQ[2] = kz * PQz;
    g.T = rho * (PQx * PQx + PQy * PQy + PQz * PQz);
    // 2 pi^(5/2) / (zeta eta sqrt(zeta+eta)), with 1/zeta and 1/eta folded into Kc
    g.pref = 34.98683665524972497 * B.Kc * K.Kc * sqrt(ize);
    g.roz = ke;  // rho / zeta
    g.roe = kz;  // rho / eta
    g.i2ze = 0.5 * ize;
}

// F_0..F_L at T, each multiplied by pref.
//   T < ERI_BT_TMAX: Taylor expansion of F_L about the nearest table point,
//     F_L(T_k + d) = sum_j F_{L+j}(T_k) (-d)^j / j!, |d| <= 1/64, seven terms
//     (remainder below 5e-17 relative), exp(-T) = exp(-T_k) exp(-d) by a
//     degree-7 polynomial, then the downward recursion
//     F_m = (2 T F_{m+1} + exp(-T)) / (2m + 1).
//   T >= ERI_BT_TMAX: F_0 = sqrt(pi / T) / 2 (erfc(6) < 3e-17) and the upward
//     recursion F_{m+1} = ((2m+1) F_m - exp(-T)) / (2T).
//   TAB_EXP: exp(-T) of the upward branch comes from the same table instead of
//     exp(): T = 2^j t with t in [TMAX/2, TMAX), exp(-T) = exp(-t)^(2^j).  The
//     j squarings scale its relative error by 2^j (j <= 5 until exp(-T)
//     underflows, near T = 745), while the share of exp(-T) in F_m falls from
//     at most 1e-4 (m = 16, T = 36) to below 1e-15 at T = 72, so F_m keeps
//     full precision.  It takes a few more instructions than exp() but no
//     constants of its own, which a kernel whose loop holds exp() keeps in
//     registers across the whole loop.

// exp(-t) for t in [0, ERI_BT_TMAX]: the table point exp(-T_k) times the
// degree-7 Taylor polynomial of exp(-d), |d| <= 1/64 (remainder below 4e-19).
__device__ __forceinline__ double eri_exp_tab(const double* __restrict__ row, double d)
{
    double ed = 1.0 - d * (1.0 / 7.0);
    ed = 1.0 - d * (1.0 / 6.0) * ed;
    ed = 1.0 - d * (1.0 / 5.0) * ed;
    ed = 1.0 - d * (1.0 / 4.0) * ed;
    ed = 1.0 - d * (1.0 / 3.0) * ed;
    ed = 1.0 - d * (1.0 / 2.0) * ed;
    ed = 1.0 - d * ed;
    return row[0] * ed;
}

template <int L, bool TAB_EXP = false>
__device__ __forceinline__ void eri_boys(double T, double pref, const double* __restrict__ tab, double* F)
{
    if (T < (double)ERI_BT_TMAX) {
        const int k = (int)(T * (double)ERI_BT_PER_UNIT + 0.5);
        const double d = T - (double)k * (1.0 / ERI_BT_PER_UNIT);
        const double* row = tab + (size_t)k * ERI_BT_COLS;
        double f = row[1 + L + 6];
        f = row[1 + L + 5] - d * (1.0 / 6.0) * f;
        f = row[1 + L + 4] - d * (1.0 / 5.0) * f;
        f = row[1 + L + 3] - d * (1.0 / 4.0) * f;
        f = row[1 + L + 2] - d * (1.0 / 3.0) * f;
        f = row[1 + L + 1] - d * (1.0 / 2.0) * f;
        f = row[1 + L + 0] - d * f;
        const double e = eri_exp_tab(row, d);
        F[L] = f;
#pragma unroll
        for (int m = L - 1; m >= 0; --m) F[m] = (2.0 * T * F[m + 1] + e) * (1.0 / (2 * m + 1));
    } else {
        double e;
        if (TAB_EXP) {
            double t = T;
            int j = 0;
            while (t >= (double)ERI_BT_TMAX) {
                t *= 0.5;
                ++j;
            }
            const int k = (int)(t * (double)ERI_BT_PER_UNIT + 0.5);
            e = eri_exp_tab(tab + (size_t)k * ERI_BT_COLS, t - (double)k * (1.0 / ERI_BT_PER_UNIT));
            for (int i = 0; i < j; ++i) e *= e;
        } else {
            e = exp(-T);
        }
        const double it = 1.0 / T;
        F[0] = 0.88622692545275801365 * sqrt(it);  // sqrt(pi)/2 / sqrt(T)
#pragma unroll
        for (int m = 0; m < L; ++m) F[m + 1] = ((2 * m + 1) * F[m] - e) * (0.5 * it);
    }
#pragma unroll
    for (int m = 0; m <= L; ++m) F[m] *= pref;
}

// Output blocks are written once and not read back by the kernel: streaming
// (non-temporal) stores keep them from displacing inputs in the caches.
__device__ __forceinline__ void eri_out(double* p, double v) { __builtin_nontemporal_store(v, p); }

// Plain (cached) output store.  Where several waves write interleaved parts of
// one block (the multi-quartet workgroups), streaming stores leave partial
// lines that reach HBM more than once (measured: 1.33x the output bytes);
// through the cache the partial lines merge first.
__device__ __forceinline__ void eri_out_merged(double* p, double v) { *p = v; }

// A value that every lane of the wave holds identically (one quartet per
// wave): reading it from the first lane lets the compiler keep it in scalar
// registers and use it as a scalar operand, freeing two VGPRs per value.
__device__ __forceinline__ double eri_uniform(double x)
{
    const long long b = __double_as_longlong(x);
    const int lo = __builtin_amdgcn_readfirstlane((int)(b & 0xffffffffLL));
    const int hi = __builtin_amdgcn_readfirstlane((int)(b >> 32));
    return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}

// Read a double held by another lane of the same wave (ds_bpermute, byte address = lane * 4).
__device__ __forceinline__ double eri_bperm(int byte_addr, double v)
{
    const int lo = __double2loint(v), hi = __double2hiint(v);
    const int rlo = __builtin_amdgcn_ds_bpermute(byte_addr, lo);
    const int rhi = __builtin_amdgcn_ds_bpermute(byte_addr, hi);
    return __hiloint2double(rhi, rlo);
}

// Buffer-instruction access to a workgroup's scratch slice: byte offset =
// per-lane VGPR offset + uniform scalar offset (memory-tier kernels).
typedef unsigned int eri_u2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ double eri_bld(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    return __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}

__device__ __forceinline__ void eri_bst(__amdgpu_buffer_rsrc_t r, int voff, int soff, double v)
{
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(eri_u2, v), r, voff, soff, 0);
}
