// Host runtime and support kernels behind the C ABI of include/eri.h.
//
// Source: "FusionRCG: Orchestrating Recursive Computation Graphs across GPU
// Memory Hierarchies".  The page's runtime (section III-C, Algorithm 2) takes
// shell quartets with their primitives {(alpha_i, c_i)}, forms Gaussian-pair
// data, evaluates one angular-momentum class per kernel and
// scatters into J.  Everything here runs on the device except argument
// validation and the small class-block bookkeeping the host needs to launch.
// The library allocates no device memory: plans and calls work in workspaces
// the caller provides (sizes from the same calls with a NULL workspace); the
// Boys table and the FMA-rate sink are file-scope device arrays.
#include <hip/hip_runtime.h>
#include <hipcub/hipcub.hpp>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "eri_device.h"
#include "eri.h"
#include "generated/eri_sph_table.h"

namespace {

thread_local std::string g_last_error;

struct HipFail {
    hipError_t e;
};

#define HIP_CHECK(x)                                                                                  \
    do {                                                                                              \
        hipError_t _e = (x);                                                                          \
        if (_e != hipSuccess) {                                                                       \
            g_last_error = std::string(#x) + ": " + hipGetErrorString(_e);                            \
            throw HipFail{_e};                                                                        \
        }                                                                                             \
    } while (0)

// class ids of quartets whose shells reach l = ERI_MAX_L + 1 (the raised-shell
// classes of the derivative integrals): 21 pair classes, 231 class ids
constexpr int ERI_NCLASS = 231;

inline int ncart(int l) { return (l + 1) * (l + 2) / 2; }
inline int nsph(int l) { return 2 * l + 1; }
inline int nfun(int l, bool sph) { return sph ? nsph(l) : ncart(l); }
inline int pair_class(int la, int lb) { return la * (la + 1) / 2 + lb; }  // la >= lb
__host__ __device__ inline int class_id_of(int pcb, int pck) { return pcb * (pcb + 1) / 2 + pck; }

__host__ __device__ inline int d_pair_class(int la, int lb)
{
    return la >= lb ? la * (la + 1) / 2 + lb : lb * (lb + 1) / 2 + la;
}

// ---------------------------------------------------------------------------
// Boys table (host, long double), one copy in every device's memory
// ---------------------------------------------------------------------------
// F_M(T) by its power series in long double, F_M = exp(-T) sum_k (2T)^k /
// ((2M+1)(2M+3)...(2M+2k+1)), then the downward recursion to F_0.
void boys_row_host(long double T, int M, long double *F)
{
    long double term = 1.0L / (2 * M + 1), sum = term;
    for (int k = 1; k < 2000; ++k) {
        term *= 2.0L * T / (2 * M + 2 * k + 1);
        sum += term;
        if (term < 1e-22L * sum && k > T) break;
    }
    long double e = expl(-T);
    F[M] = e * sum;
    for (int m = M - 1; m >= 0; --m) F[m] = (2.0L * T * F[m + 1] + e) / (2 * m + 1);
}

}  // namespace

// file-scope device arrays (each device holds its own copy)
__device__ double g_boys_tab[ERI_BT_ROWS * ERI_BT_COLS];
__device__ double g_fma_sink[1];

namespace {

std::mutex g_boys_mu;
std::vector<double *> g_boys_dev;
std::vector<double> g_boys_host;

// the table on the current device (filled once per device)
double *boys_table(int device)
{
    std::lock_guard<std::mutex> lk(g_boys_mu);
    if ((int)g_boys_dev.size() <= device) g_boys_dev.resize(device + 1, nullptr);
    if (g_boys_dev[device]) return g_boys_dev[device];
    if (g_boys_host.empty()) {
        g_boys_host.resize((size_t)ERI_BT_ROWS * ERI_BT_COLS);
        long double F[ERI_BT_MMAX + 1];
        for (int k = 0; k < ERI_BT_ROWS; ++k) {
            long double T = (long double)k / ERI_BT_PER_UNIT;
            boys_row_host(T, ERI_BT_MMAX, F);
            g_boys_host[(size_t)k * ERI_BT_COLS] = (double)expl(-T);
            for (int m = 0; m <= ERI_BT_MMAX; ++m) g_boys_host[(size_t)k * ERI_BT_COLS + 1 + m] = (double)F[m];
        }
    }
    HIP_CHECK(hipMemcpyToSymbol(HIP_SYMBOL(g_boys_tab), g_boys_host.data(), g_boys_host.size() * sizeof(double), 0,
                                hipMemcpyHostToDevice));
    double *d = nullptr;
    HIP_CHECK(hipGetSymbolAddress((void **)&d, HIP_SYMBOL(g_boys_tab)));
    g_boys_dev[device] = d;
    return d;
}

const EriClassEntry *find_class(int cid, bool sph)
{
    for (int i = 0; i < eri_class_table_size; ++i)
        if (eri_class_table[i].class_id == cid && eri_class_table[i].spherical == (sph ? 1 : 0))
            return &eri_class_table[i];
    return nullptr;
}

// ---------------------------------------------------------------------------
// support kernels
// ---------------------------------------------------------------------------

// Contraction coefficients on normalised primitives: c_k N(alpha_k, l), then the
// contracted x^l component scaled to unit norm (see include/eri.h).
__global__ void k_normalize(int nshell, const int *l, const int *nprim, const int *off, const double *exps,
                            const double *coefs, double *out, int raw)
{
    const int s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= nshell) return;
    const int L = l[s], K = nprim[s], o = off[s];
    if (raw) {
        for (int k = 0; k < K; ++k) out[o + k] = coefs[o + k];
        return;
    }
    double df = 1.0;  // (2L-1)!!
    for (int t = 2 * L - 1; t > 1; t -= 2) df *= t;
    for (int k = 0; k < K; ++k) {
        const double a = exps[o + k];
        out[o + k] = coefs[o + k] * pow(2.0 * a / M_PI, 0.75) * pow(4.0 * a, 0.5 * L) / sqrt(df);
    }
    double norm2 = 0.0;
    for (int k = 0; k < K; ++k)
        for (int q = 0; q < K; ++q) {
            const double p = exps[o + k] + exps[o + q];
            norm2 += out[o + k] * out[o + q] * pow(M_PI / p, 1.5) * df / pow(2.0 * p, L);
        }
    const double f = 1.0 / sqrt(norm2);
    for (int k = 0; k < K; ++k) out[o + k] *= f;
}

// Primitive-pair screening of screened plans.  A primitive pair (alpha of
// shell A, beta of shell B) enters the plan when its Gaussian-product exponent
// q = alpha beta / (alpha + beta) |AB|^2 is at most PRIM_QMAX, i.e. its factor
// exp(-q) is at least 1.3e-100; a shell pair with no such primitive pair keeps
// its first one.  A dropped pair's share of any integral is below 1e-100 times
// its normalisation and polynomial factors, far under the rounding of the
// result.  q is formed as ((alpha beta) / (alpha + beta)) AB2 with AB2 =
// (dx dx + dy dy) + dz dz in correctly rounded steps and no fused operations,
// on the host (bucket sizes) and on the device (records) alike, so both take
// the same decisions.
constexpr double PRIM_QMAX = 230.0;

__host__ __device__ inline double prim_q(double al, double be, double dx, double dy, double dz)
{
#pragma clang fp contract(off)
    const double AB2 = (dx * dx + dy * dy) + dz * dz;
    return (al * be) / (al + be) * AB2;
}

// number of primitive pairs of shells a, b a screened plan keeps
inline int prim_pairs_kept(const double *cen, const int *off, const double *exps, int a, int b)
{
    const double dx = cen[3 * a] - cen[3 * b], dy = cen[3 * a + 1] - cen[3 * b + 1], dz = cen[3 * a + 2] - cen[3 * b + 2];
    int n = 0;
    for (int ia = off[a]; ia < off[a + 1]; ++ia)
        for (int ib = off[b]; ib < off[b + 1]; ++ib)
            n += prim_q(exps[ia], exps[ib], dx, dy, dz) <= PRIM_QMAX ? 1 : 0;
    return n > 0 ? n : 1;
}

// Primitive-pair records for every shell pair (the page's Gaussian-pair step);
// screened plans keep the primitive pairs prim_pairs_kept counts, in
// (alpha, beta) order.
__global__ void k_pair_data(int npairs, const int4 *pinfo, const double *cen, const int *off,
                            const double *exps, const double *cn, int screened, double *ppd)
{
    const int p = blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= npairs) return;
    const int4 pi = pinfo[p];
    const int a = pi.x, b = pi.y;
    const double Ax = cen[3 * a], Ay = cen[3 * a + 1], Az = cen[3 * a + 2];
    const double Bx = cen[3 * b], By = cen[3 * b + 1], Bz = cen[3 * b + 2];
    const double AB2 = (Ax - Bx) * (Ax - Bx) + (Ay - By) * (Ay - By) + (Az - Bz) * (Az - Bz);
    const int Ka = off[a + 1] - off[a], Kb = off[b + 1] - off[b];
    // primitive pairs within the screen; a shell pair with none keeps its first
    int within = 0;
    if (screened)
        for (int ia = 0; ia < Ka; ++ia)
            for (int ib = 0; ib < Kb; ++ib)
                within += prim_q(exps[off[a] + ia], exps[off[b] + ib], Ax - Bx, Ay - By, Az - Bz) <= PRIM_QMAX ? 1 : 0;
    int n = 0;
    for (int ia = 0; ia < Ka; ++ia)
        for (int ib = 0; ib < Kb; ++ib) {
            const double al = exps[off[a] + ia], be = exps[off[b] + ib];
            if (screened) {
                const bool keep = within == 0 ? (ia == 0 && ib == 0)
                                              : prim_q(al, be, Ax - Bx, Ay - By, Az - Bz) <= PRIM_QMAX;
                if (!keep) continue;
            }
            if (n >= pi.w) continue;  // never past the records the plan reserved for this pair
            const double z = al + be, iz = 1.0 / z;
            const double Px = (al * Ax + be * Bx) * iz, Py = (al * Ay + be * By) * iz, Pz = (al * Az + be * Bz) * iz;
            double *r = ppd + (size_t)(pi.z + n++) * ERI_PP_STRIDE;
            r[0] = z;
            r[1] = iz;
            r[2] = Px;
            r[3] = Py;
            r[4] = Pz;
            // P - A = beta (B - A) / zeta: exact zero for a one-centre pair
            r[5] = be * (Bx - Ax) * iz;
            r[6] = be * (By - Ay) * iz;
            r[7] = be * (Bz - Az) * iz;
            r[8] = cn[off[a] + ia] * cn[off[b] + ib] * exp(-al * be * iz * AB2) * iz;
            r[9] = 0.0;
        }
    // The host counted the same kept pairs with the same arithmetic, so n equals
    // pi.w; should it fall short, the missing records repeat the first with
    // zero weight instead of being left unwritten.
    const double *r0 = ppd + (size_t)pi.z * ERI_PP_STRIDE;
    for (; n > 0 && n < pi.w; ++n) {
        double *r = ppd + (size_t)(pi.z + n) * ERI_PP_STRIDE;
        for (int f = 0; f < ERI_PP_STRIDE; ++f) r[f] = f == 8 ? 0.0 : r0[f];
    }
}

__device__ inline void canonical4(const int *l, int &i, int &j, int &k, int &m, int &perm)
{
    perm = 0;
    if (l[i] < l[j]) {
        int t = i; i = j; j = t;
        perm |= 1;
    }
    if (l[k] < l[m]) {
        int t = k; k = m; m = t;
        perm |= 2;
    }
    if (d_pair_class(l[i], l[j]) < d_pair_class(l[k], l[m])) {
        int t = i; i = k; k = t;
        t = j; j = m; m = t;
        perm |= 4;
    }
}

// Explicit lists: sort key (class, K_bra, K_ket, position).
__global__ void k_explicit_keys(int64_t nq, const int *q, const int *l, const int *nprim, uint64_t *keys,
                                int64_t *pos)
{
    const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= nq) return;
    int i = q[4 * x], j = q[4 * x + 1], k = q[4 * x + 2], m = q[4 * x + 3], perm;
    canonical4(l, i, j, k, m, perm);
    const uint64_t cid = class_id_of(d_pair_class(l[i], l[j]), d_pair_class(l[k], l[m]));
    const uint64_t kb = (uint64_t)(nprim[i] * nprim[j]), kk = (uint64_t)(nprim[k] * nprim[m]);
    keys[x] = (cid << 56) | (kb << 48) | (kk << 40) | (uint64_t)x;
    pos[x] = x;
}

__global__ void k_explicit_fill(int64_t nq, const int64_t *pos, const int *q, const int *l, const int *nprim,
                                int *qmap, int *qbra, int *qket, int4 *pinfo)
{
    const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= nq) return;
    const int64_t x = pos[s];
    int i = q[4 * x], j = q[4 * x + 1], k = q[4 * x + 2], m = q[4 * x + 3], perm;
    canonical4(l, i, j, k, m, perm);
    qmap[5 * s] = i;
    qmap[5 * s + 1] = j;
    qmap[5 * s + 2] = k;
    qmap[5 * s + 3] = m;
    qmap[5 * s + 4] = perm;
    qbra[s] = (int)(2 * s);
    qket[s] = (int)(2 * s + 1);
    pinfo[2 * s] = make_int4(i, j, 0, nprim[i] * nprim[j]);
    pinfo[2 * s + 1] = make_int4(k, m, 0, nprim[k] * nprim[m]);
}

// start of each class in the sorted keys (lower bound of class << 56), and the
// end of its uncontracted prefix (K_bra = K_ket = 1 sort first in a class)
__global__ void k_class_starts(int64_t n, const uint64_t *keys, int64_t *starts, int64_t *k1_end, int nclass)
{
    const int c = blockIdx.x * blockDim.x + threadIdx.x;
    if (c > nclass) return;
    for (int pass = 0; pass < 2; ++pass) {
        const uint64_t target = pass == 0 ? ((uint64_t)c << 56)
                                          : (((uint64_t)c << 56) | ((uint64_t)1 << 48) | ((uint64_t)2 << 40));
        int64_t lo = 0, hi = n;
        while (lo < hi) {
            int64_t mid = (lo + hi) / 2;
            if (keys[mid] < target) lo = mid + 1;
            else hi = mid;
        }
        if (pass == 0) starts[c] = lo;
        else k1_end[c] = lo;
    }
}

__global__ void k_copy_w(int n, const int4 *pinfo, int *w)
{
    const int p = blockIdx.x * blockDim.x + threadIdx.x;
    if (p < n) w[p] = pinfo[p].w;
}

__global__ void k_set_z(int n, int4 *pinfo, const int *z)
{
    const int p = blockIdx.x * blockDim.x + threadIdx.x;
    if (p < n) pinfo[p].z = z[p];
}

// All pairs i >= j, oriented so that l_a >= l_b (equal l: a = i), with the
// primitive pairs a screened plan keeps (counted on the host, kept[p]).
__global__ void k_all_pairs(int nshell, const int *l, const int *kept, int4 *pinfo, uint64_t *pc_key, int *pidx)
{
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t np = (int64_t)nshell * (nshell + 1) / 2;
    if (p >= np) return;
    int i = (int)floor((sqrt(8.0 * (double)p + 1.0) - 1.0) * 0.5);
    while ((int64_t)i * (i + 1) / 2 > p) --i;
    while ((int64_t)(i + 1) * (i + 2) / 2 <= p) ++i;
    const int j = (int)(p - (int64_t)i * (i + 1) / 2);
    int a = i, b = j;
    if (l[i] < l[j]) {
        a = j;
        b = i;
    }
    pinfo[p] = make_int4(a, b, 0, kept[p]);
    pc_key[p] = (uint64_t)d_pair_class(l[a], l[b]);
    pidx[p] = (int)p;
}

// Sub-pairs for the Schwarz diagonals: pair p's kept primitive-pair records
// split into ceil(K / SCHWARZ_SUBK) consecutive runs, sub-pair kpo[p] + i
// holding records i SCHWARZ_SUBK ... (as many as remain).  The diagonal block
// (p|p) is the sum of the blocks (p_i|p_j) over all sub-pair pairs (the
// integral is linear in the primitive pairs of each side), and a quartet of
// sub-pairs has at most SCHWARZ_SUBK^2 primitive quartets, so a pair with a
// long contraction no longer runs as one long loop on one lane.
constexpr int SCHWARZ_SUBK = 6;

__global__ void k_sub_pairs(int np, const int4 *pinfo, const int64_t *kpo, int4 *sub)
{
    const int p = blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= np) return;
    const int4 pi = pinfo[p];
    const int64_t o = kpo[p];
    const int k = (pi.w + SCHWARZ_SUBK - 1) / SCHWARZ_SUBK;
    for (int i = 0; i < k; ++i)
        sub[o + i] = make_int4(pi.x, pi.y, pi.z + i * SCHWARZ_SUBK, min(SCHWARZ_SUBK, pi.w - i * SCHWARZ_SUBK));
}

// S of each pair of a batch: the diagonal of the sum of its k^2 sub-pair blocks
// (block offset boff[t], in units of blocks of nab^2), summed in (i, j) order
__global__ void k_schwarz_sum_max(int n, const int *pairs, const int *ksub, const int64_t *boff, const double *blk,
                                  int nab, double *S)
{
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n) return;
    const int k2 = ksub[t] * ksub[t];
    const double *B = blk + (size_t)boff[t] * nab * nab;
    double mx = 0.0;
    for (int u = 0; u < nab; ++u) {
        double v = 0.0;
        for (int x = 0; x < k2; ++x) v += B[(size_t)x * nab * nab + (size_t)u * nab + u];
        mx = fmax(mx, fabs(v));
    }
    S[pairs[t]] = mx;
}

__global__ void k_desc_keys(int n, const int *pidx, const double *S, uint64_t *key)
{
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n) return;
    const double s = S[pidx[t]];
    key[t] = ~(uint64_t)__double_as_longlong(s);  // S >= 0: bit order = value order
}

__global__ void k_bucket_keys(int n, const int *pidx, const int *l, const int4 *pinfo, uint64_t *key)
{
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n) return;
    const int4 pi = pinfo[pidx[t]];
    key[t] = ((uint64_t)d_pair_class(l[pi.x], l[pi.y]) << 16) | (uint64_t)pi.w;
}

__global__ void k_heads(int n, const uint64_t *key, int *head)
{
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n) return;
    head[t] = (t == 0 || key[t] != key[t - 1]) ? 1 : 0;
}

__global__ void k_bucket_table(int n, const uint64_t *key, const int *head, const int *hscan, int *bstart,
                               uint64_t *bkey)
{
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n) return;
    if (head[t]) {
        bstart[hscan[t]] = t;
        bkey[hscan[t]] = key[t];
    }
}

struct BlockDesc {
    int bra_start, bra_n;  // sorted-pair range of the bra bucket
    int ket_start, ket_n;  // sorted-pair range of the ket bucket
    int same;              // bra bucket == ket bucket
    int64_t entry_base;    // first (block, bra) entry
};

// per (block, bra rank): number of surviving kets, fl(S_b * S_k) >= tau2
__global__ void k_count(int64_t nentries, const BlockDesc *blocks, int nblocks, const int *porder, const double *S,
                        double tau2, int64_t *cnt)
{
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= nentries) return;
    int lo = 0, hi = nblocks;  // last block with entry_base <= e
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (blocks[mid].entry_base <= e) lo = mid;
        else hi = mid;
    }
    const BlockDesc bd = blocks[lo];
    const int r = (int)(e - bd.entry_base);
    const double sb = S[porder[bd.bra_start + r]];
    // kets sorted by S descending: the survivors are a prefix
    int a = 0, b = bd.ket_n;
    while (a < b) {
        int mid = (a + b) / 2;
        const double prod = __dmul_rn(sb, S[porder[bd.ket_start + mid]]);
        if (prod >= tau2) a = mid + 1;
        else b = mid;
    }
    int64_t c = a;
    if (bd.same) c = c > r ? c - r : 0;
    cnt[e] = c;
}

// Plan slots [s0, s0 + m) of an implicit screened plan -> bra and ket pair
// (and, when qmap is given, the index-map rows).  The slot's entry (block,
// bra rank) is the last entry whose offset is <= the slot: entries without
// survivors share the next entry's offset.
__global__ void k_expand(int64_t s0, int64_t m, int64_t nent, const int64_t *off, const BlockDesc *blocks,
                         int nblocks, const int *porder, const int4 *pinfo, const int *pair_i, int *qbra, int *qket,
                         int *qmap)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= m) return;
    const int64_t s = s0 + t;
    int64_t lo = 0, hi = nent;
    while (hi - lo > 1) {
        const int64_t mid = (lo + hi) / 2;
        if (off[mid] <= s) lo = mid;
        else hi = mid;
    }
    const int64_t e = lo;
    int blo = 0, bhi = nblocks;
    while (bhi - blo > 1) {
        const int mid = (blo + bhi) / 2;
        if (blocks[mid].entry_base <= e) blo = mid;
        else bhi = mid;
    }
    const BlockDesc bd = blocks[blo];
    const int r = (int)(e - bd.entry_base);
    const int pb = porder[bd.bra_start + r];
    const int pk = porder[bd.ket_start + (bd.same ? r : 0) + (int)(s - off[e])];
    if (qbra) qbra[t] = pb;
    if (qket) qket[t] = pk;
    if (qmap) {
        const int4 ib = pinfo[pb], ik = pinfo[pk];
        int *row = qmap + 5 * t;
        row[0] = ib.x;
        row[1] = ib.y;
        row[2] = ik.x;
        row[3] = ik.y;
        row[4] = (ib.x != pair_i[pb] ? 1 : 0) | ((ik.x != pair_i[pk] ? 1 : 0) << 1) | ((pb < pk ? 1 : 0) << 2);
    }
}

__global__ void k_zero_mat(int n, double *A, int lda)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (int64_t)n * n) return;
    const int i = (int)(t / n), j = (int)(t - (int64_t)i * n);
    A[(size_t)i * lda + j] = 0.0;
}

// chunk entries: (pair, offset of its contribution vector) for both sides of
// every quartet; a quartet of two equal pairs has one side only
// (contribution vectors at cb offset base + s (nab + ncd), entries from ekey/eoff on)
__global__ void k_chunk_entries(int m, const int *qbra, const int *qket, int nab, int ncd, int none, int64_t base,
                                int *ekey, int *eoff)
{
    const int s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= m) return;
    const int off = (int)(base + (int64_t)s * (nab + ncd));  // below the lane's CB <= 2^26 doubles
    ekey[2 * s] = qbra[s];
    eoff[2 * s] = off;
    const bool two = qbra[s] != qket[s];
    ekey[2 * s + 1] = two ? qket[s] : none;  // sorts last, never read
    eoff[2 * s + 1] = two ? off + nab : -1;
}

// Sum of the entries e0, e0+1, ..., e1-1 of a run of contribution vectors of
// length n (n <= blockDim.x), in a fixed order: the block splits into
// S = blockDim.x / n slices, slice k adds the entries e0 + k, e0 + k + S, ...
// in entry order, and thread v < n then adds the S partial sums in slice
// order.  Deterministic for a given blockDim; the result is left in part[v].
__device__ __forceinline__ void run_sum(int n, int64_t e0, int64_t e1, const int *eoff, const double *cb,
                                        double *part)
{
    const int S = blockDim.x / n;
    const int v = threadIdx.x % n, sl = threadIdx.x / n;
    double acc = 0.0;
    if (sl < S)
        for (int64_t e = e0 + sl; e < e1; e += S) acc += cb[eoff[e] + v];
    part[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x < n) {
        double t = 0.0;
        for (int k = 0; k < S; ++k) t += part[k * n + threadIdx.x];
        part[threadIdx.x] = t;  // slot threadIdx.x < n was read only by this thread
    }
}

constexpr int RUN_THREADS = 256;

// one workgroup per run of equal pairs in the sorted chunk entries: add the
// run's contribution vectors into the J block (and its transpose)
__global__ void __launch_bounds__(RUN_THREADS) k_add_runs(const int *nruns, const int *key, const int *rstart,
                                                          const int *rlen, const int *eoff, const double *cb,
                                                          const int4 *pinfo, const int *bf, const int *nfun_sh,
                                                          int none, double *J, int ldj)
{
    __shared__ double part[RUN_THREADS];
    const int u = blockIdx.x;
    if (u >= *nruns) return;
    const int p = key[u];
    if (p == none) return;
    const int4 pi = pinfo[p];
    const int na = nfun_sh[pi.x], nb = nfun_sh[pi.y], n = na * nb;
    const int64_t e0 = rstart[u], e1 = e0 + rlen[u];
    run_sum(n, e0, e1, eoff, cb, part);
    const int v = threadIdx.x;
    if (v < n) {
        const double acc = part[v];
        const int a = v / nb, b = v - a * nb;
        J[(size_t)(bf[pi.x] + a) * ldj + bf[pi.y] + b] += acc;
        if (pi.x != pi.y) J[(size_t)(bf[pi.y] + b) * ldj + bf[pi.x] + a] += acc;
    }
}

// ---- K digestion ----------------------------------------------------------
//
// K_mu,nu = sum (mu la|nu si) D_la,si.  A unique quartet (ij|kl) stands for
// up to eight ordered shell quadruples.  Those with i in the bra's first and k
// in the ket's first position give four blocks of
//   A_ik += I D_jl,  A_jk += I D_il (i != j),  A_il += I D_jk (k != l),
//   A_jl += I D_ik (i != j, k != l),
// each contracted over the other two indices; the other four quadruples give
// the transposed blocks, so K = A + A^T for a symmetric D.  When the bra and
// ket pairs are the same pair, the transposed quadruples are the same as the
// first four: those quartets count one half in A.

// per quartet: the four blocks V1 (na x nc), V2 (nb x nc), V3 (na x nd), V4 (nb x nd),
// one thread per element of the m quartets' vectors (w elements per quartet)
__global__ void k_kdigest_rows(int64_t n_out, int na, int nb, int nc, int nd, const int *qbra, const int *qket,
                               const int4 *pinfo, const int *bf, const double *I, const double *D, int ldd,
                               double *kv)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n_out) return;
    const int w1 = na * nc, w2 = nb * nc, w3 = na * nd, w4 = nb * nd, w = w1 + w2 + w3 + w4;
    const int64_t q = t / w;
    int u = (int)(t - q * w);
    const int pb = qbra[q], pk = qket[q];
    const int4 ib = pinfo[pb], ik = pinfo[pk];
    const int i0 = bf[ib.x], j0 = bf[ib.y], k0 = bf[ik.x], l0 = bf[ik.y];
    const bool dij = ib.x != ib.y, dkl = ik.x != ik.y;
    const double wt = pb == pk ? 0.5 : 1.0;
    const double *blk = I + (size_t)q * (na * nb) * (nc * nd);
    double acc = 0.0;
    if (u < w1) {
        const int a = u / nc, c = u - a * nc;
        for (int b = 0; b < nb; ++b)
            for (int d = 0; d < nd; ++d) acc += blk[((size_t)(a * nb + b) * nc + c) * nd + d] * D[(size_t)(j0 + b) * ldd + l0 + d];
    } else if ((u -= w1) < w2) {
        const int b = u / nc, c = u - b * nc;
        if (dij)
            for (int a = 0; a < na; ++a)
                for (int d = 0; d < nd; ++d) acc += blk[((size_t)(a * nb + b) * nc + c) * nd + d] * D[(size_t)(i0 + a) * ldd + l0 + d];
    } else if ((u -= w2) < w3) {
        const int a = u / nd, d = u - a * nd;
        if (dkl)
            for (int b = 0; b < nb; ++b)
                for (int c = 0; c < nc; ++c) acc += blk[((size_t)(a * nb + b) * nc + c) * nd + d] * D[(size_t)(j0 + b) * ldd + k0 + c];
    } else {
        u -= w3;
        const int b = u / nd, d = u - b * nd;
        if (dij && dkl)
            for (int a = 0; a < na; ++a)
                for (int c = 0; c < nc; ++c) acc += blk[((size_t)(a * nb + b) * nc + c) * nd + d] * D[(size_t)(i0 + a) * ldd + k0 + c];
    }
    kv[t] = wt * acc;
}

// chunk entries for K: (target shell block s1 * nshell + s2, offset of the block's
// vector) for the four blocks of every quartet; blocks a quartet does not have
// get a key that sorts last
__global__ void k_kchunk_entries(int m, const int *qbra, const int *qket, const int4 *pinfo, int nshell, int na,
                                 int nb, int nc, int nd, int *ekey, int *eoff)
{
    const int q = blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= m) return;
    const int4 ib = pinfo[qbra[q]], ik = pinfo[qket[q]];
    const bool dij = ib.x != ib.y, dkl = ik.x != ik.y;
    const int base = q * (na * nc + nb * nc + na * nd + nb * nd);  // below the lane's CB <= 2^26 doubles
    const int none = nshell * nshell;  // above every block key
    ekey[4 * q] = ib.x * nshell + ik.x;
    eoff[4 * q] = base;
    ekey[4 * q + 1] = dij ? ib.y * nshell + ik.x : none;
    eoff[4 * q + 1] = base + na * nc;
    ekey[4 * q + 2] = dkl ? ib.x * nshell + ik.y : none;
    eoff[4 * q + 2] = base + na * nc + nb * nc;
    ekey[4 * q + 3] = (dij && dkl) ? ib.y * nshell + ik.y : none;
    eoff[4 * q + 3] = base + na * nc + nb * nc + na * nd;
}

// one workgroup per run of equal target blocks: add the run's vectors into A
__global__ void __launch_bounds__(RUN_THREADS) k_add_runs_K(const int *nruns, const int *key, const int *rstart,
                                                            const int *rlen, const int *eoff, const double *kv,
                                                            int nshell, const int *bf, const int *nfun_sh, double *A,
                                                            int lda)
{
    __shared__ double part[RUN_THREADS];
    const int u = blockIdx.x;
    if (u >= *nruns) return;
    const int k = key[u];
    if (k == nshell * nshell) return;
    const int s1 = k / nshell, s2 = k - s1 * nshell;
    const int n1 = nfun_sh[s1], n2 = nfun_sh[s2];
    const int64_t e0 = rstart[u], e1 = e0 + rlen[u];
    run_sum(n1 * n2, e0, e1, eoff, kv, part);
    const int v = threadIdx.x;
    if (v < n1 * n2) {
        const int x = v / n2, y = v - x * n2;
        A[(size_t)(bf[s1] + x) * lda + bf[s2] + y] += part[v];
    }
}

// K = A + A^T
__global__ void k_sym_add(int n, const double *A, int lda, double *K, int ldk)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (int64_t)n * n) return;
    const int x = (int)(t / n), y = (int)(t - (int64_t)x * n);
    K[(size_t)x * ldk + y] = A[(size_t)x * lda + y] + A[(size_t)y * lda + x];
}

__global__ void k_pair_hi(int np, const int4 *pinfo, int *hi)
{
    const int p = blockIdx.x * blockDim.x + threadIdx.x;
    if (p < np) hi[p] = max(pinfo[p].x, pinfo[p].y);
}

__global__ void k_gather_i64(int n, const int64_t *src, const int64_t *idx, int64_t *dst)
{
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t < n) dst[t] = src[idx[t]];
}

// ---- J digestion ----------------------------------------------------------

// Per quartet of one class block: vb[ab] = sum_cd I[ab,cd] D~_cd and, for
// distinct pairs, vk[cd] = sum_ab I[ab,cd] D~_ab, with D~ = D x 2 for a pair of
// two different shells (the 8-fold symmetry factors).  One thread per element
// of the m quartets' vectors (nab + ncd per quartet, stored back to back).
__global__ void k_digest_rows(int64_t n_out, int na, int nb, int nc, int nd, const int *qbra, const int *qket,
                              const int4 *pinfo, const int *bf, const double *I, const double *D, int ldd,
                              double *cb)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n_out) return;
    const int nab = na * nb, ncd = nc * nd, w = nab + ncd;
    const int64_t q = t / w;
    const int r = (int)(t - q * w);
    const int pb = qbra[q], pk = qket[q];
    const double *blk = I + (size_t)q * nab * ncd;
    double s = 0.0;
    if (r < nab) {
        const int4 ik = pinfo[pk];
        const int c0 = bf[ik.x], d0 = bf[ik.y];
        const double *row = blk + (size_t)r * ncd;
        for (int c = 0; c < nc; ++c)
            for (int d = 0; d < nd; ++d) s += row[c * nd + d] * D[(size_t)(c0 + c) * ldd + d0 + d];
        s = (ik.x != ik.y ? 2.0 : 1.0) * s;
    } else {
        const int4 ib = pinfo[pb];
        const int cd = r - nab;
        if (pb != pk) {
            const int a0 = bf[ib.x], b0 = bf[ib.y];
            for (int a = 0; a < na; ++a)
                for (int b = 0; b < nb; ++b) s += blk[(size_t)(a * nb + b) * ncd + cd] * D[(size_t)(a0 + a) * ldd + b0 + b];
        }
        s = (ib.x != ib.y ? 2.0 : 1.0) * s;
    }
    cb[t] = s;
}

// ---------------------------------------------------------------------------
// First derivatives with respect to the centres
// ---------------------------------------------------------------------------
// d/dA_i of a primitive Cartesian Gaussian centred at A raises and lowers its
// angular momentum: 2 alpha phi_(a+1_i) - a_i phi_(a-1_i).  Contracted, the
// derivative block of (ab|cd) with respect to A_i is therefore
//   (a+1_i b|cd) over the shell a' (l+1, coefficients 2 alpha c)
//   - a_i (a-1_i b|cd) over the shell a'' (l-1, coefficients c),
// with c the normalised coefficients of a, both on raw monomials.  The class
// kernels compute those neighbouring integrals on an auxiliary shell set
// (three copies of every shell: itself, raised, lowered); the kernels below
// pick the two terms of every derivative element out of the auxiliary blocks
// (whose quartets the plan may have reordered: the permutation bits say how)
// and, for spherical plans, apply t^(l) to the four indices of each block.
__device__ inline int dv_ncart(int l) { return (l + 1) * (l + 2) / 2; }
__device__ inline int dv_nsph(int l) { return 2 * l + 1; }
// index of the Cartesian component (x, y, l-x-y) of a shell l: x descending, then y descending
__device__ inline int dv_cidx(int l, int x, int y)
{
    const int r = l - x;
    return r * (r + 1) / 2 + (r - y);
}
__device__ inline void dv_ctrip(int l, int i, int *t)
{
    int r = 0;
    while ((r + 1) * (r + 2) / 2 <= i) ++r;
    t[0] = l - r;
    t[1] = r - (i - r * (r + 1) / 2);
    t[2] = l - t[0] - t[1];
}

// slot of every listed auxiliary quartet, by its derivative index u (umap: the
// list's u in input order)
__global__ void k_invert_src(int64_t n, const int64_t *src, const int *umap, int64_t *slot_of)
{
    const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x < n) slot_of[umap[src[x]]] = x;
}

// output offset of every slot from the block table (blocks ordered by first slot)
__global__ void k_slot_offsets(int64_t n, int nb, const int64_t *bstart, const int64_t *bout, const int64_t *bsize,
                               int64_t *off)
{
    const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= n) return;
    int lo = 0, hi = nb - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (bstart[mid] <= x) lo = mid;
        else hi = mid - 1;
    }
    off[x] = bout[lo] + (x - bstart[lo]) * bsize[lo];
}

// tpi threads per quartet (a power of two dividing the 256 of a workgroup): its
// 12 Cartesian derivative blocks into dst + dst_off[t]
__global__ void __launch_bounds__(256) k_deriv_combine(int64_t n, int tpi, const int *rows, const int *lsh,
                                                       const int64_t *aux_slot_of, const int *aux_qmap,
                                                       const int *aux_l, const int64_t *aux_off, const double *aux,
                                                       const int64_t *dst_off, double *dst)
{
    const int64_t t = (int64_t)blockIdx.x * (256 / tpi) + threadIdx.x / tpi;
    const int lane = threadIdx.x % tpi;
    if (t >= n) return;
    int l4[4], n4[4];
    for (int k = 0; k < 4; ++k) {
        l4[k] = lsh[rows[5 * t + k]];
        n4[k] = dv_ncart(l4[k]);
    }
    const int ncar = n4[0] * n4[1] * n4[2] * n4[3];
    for (int idx = lane; idx < 12 * ncar; idx += tpi) {
        const int comp = idx / ncar, e = idx - comp * ncar;
        const int p = comp / 3, ax = comp - 3 * p;
        int ci[4], r = e;
        ci[3] = r % n4[3];
        r /= n4[3];
        ci[2] = r % n4[2];
        r /= n4[2];
        ci[1] = r % n4[1];
        ci[0] = r / n4[1];
        int tr[3];
        dv_ctrip(l4[p], ci[p], tr);
        double v = 0.0;
        for (int sg = 0; sg < 2; ++sg) {
            const int nax = tr[ax];
            if (sg == 1 && nax == 0) continue;
            const int dl = sg == 0 ? 1 : -1;
            int t2[3] = {tr[0], tr[1], tr[2]};
            t2[ax] += dl;
            int j[4] = {ci[0], ci[1], ci[2], ci[3]};
            j[p] = dv_cidx(l4[p] + dl, t2[0], t2[1]);
            const int64_t s = aux_slot_of[(t * 4 + p) * 2 + sg];
            const int perm = aux_qmap[5 * s + 4];
            int x;
            if (perm & 1) { x = j[0]; j[0] = j[1]; j[1] = x; }
            if (perm & 2) { x = j[2]; j[2] = j[3]; j[3] = x; }
            if (perm & 4) {
                x = j[0]; j[0] = j[2]; j[2] = x;
                x = j[1]; j[1] = j[3]; j[3] = x;
            }
            int m4[4];
            for (int k = 0; k < 4; ++k) m4[k] = dv_ncart(aux_l[aux_qmap[5 * s + k]]);
            const int64_t flat = ((int64_t)(j[0] * m4[1] + j[1]) * m4[2] + j[2]) * m4[3] + j[3];
            const double a = aux[aux_off[s] + flat];
            v += sg == 0 ? a : -(double)nax * a;
        }
        dst[dst_off[t] + idx] = v;
    }
}

// tpi threads per (quartet, derivative component) item (a power of two
// dividing the 256 of a workgroup): t^(l) on the four indices, ping-pong
// between the Cartesian block and a scratch block, last pass into dst.  Every
// thread of the workgroup takes part in its barriers; threads past the last
// item only wait.
__global__ void __launch_bounds__(256) k_deriv_sph(int64_t n, int tpi, const int *rows, const int *lsh, double *cart,
                                                   double *tmp, const int64_t *cart_off, const int64_t *dst_off,
                                                   double *dst)
{
    const int64_t u = (int64_t)blockIdx.x * (256 / tpi) + threadIdx.x / tpi;
    const int lane = threadIdx.x % tpi;
    const bool live = u < 12 * n;
    const int64_t t = live ? u / 12 : 0;
    const int comp = live ? (int)(u - t * 12) : 0;
    int l4[4], dims[4], ns[4];
    for (int k = 0; k < 4; ++k) {
        l4[k] = live ? lsh[rows[5 * t + k]] : 0;
        dims[k] = dv_ncart(l4[k]);
        ns[k] = dv_nsph(l4[k]);
    }
    const int ncar = dims[0] * dims[1] * dims[2] * dims[3];
    const int nsp = ns[0] * ns[1] * ns[2] * ns[3];
    double *a = cart + cart_off[t] + (int64_t)comp * ncar;
    double *b = tmp + cart_off[t] + (int64_t)comp * ncar;
    for (int pos = 0; pos < 4; ++pos) {
        int before = 1, after = 1;
        for (int k = 0; k < pos; ++k) before *= dims[k];
        for (int k = pos + 1; k < 4; ++k) after *= dims[k];
        const double *T = eri_sph_T[l4[pos]];
        const int nc = dims[pos], nsv = ns[pos];
        const double *in = (pos % 2 == 0) ? a : b;
        double *o = pos == 3 ? dst + dst_off[t] + (int64_t)comp * nsp : ((pos % 2 == 0) ? b : a);
        const int total = live ? before * nsv * after : 0;
        for (int x = lane; x < total; x += tpi) {
            const int y = x % after, rr = x / after, sv = rr % nsv, bb = rr / nsv;
            double acc = 0.0;
            for (int c = 0; c < nc; ++c) acc += T[sv * nc + c] * in[((int64_t)bb * nc + c) * after + y];
            o[x] = acc;
        }
        dims[pos] = nsv;
        __syncthreads();
    }
}


// The same transform with the item's block in LDS: the Cartesian block is read
// once, coalesced, and the four passes ping-pong between two LDS buffers of
// `stride` doubles per item (stride >= the call's largest Cartesian block;
// the caller sizes the dynamic LDS to (256 / tpi) x 2 x stride doubles).  The
// passes sum in the same order as k_deriv_sph.
__global__ void __launch_bounds__(256) k_deriv_sph_lds(int64_t n, int tpi, int stride, const int *rows, const int *lsh,
                                                       const double *cart, const int64_t *cart_off,
                                                       const int64_t *dst_off, double *dst)
{
    extern __shared__ double sm[];
    const int64_t u = (int64_t)blockIdx.x * (256 / tpi) + threadIdx.x / tpi;
    const int lane = threadIdx.x % tpi;
    const bool live = u < 12 * n;
    const int64_t t = live ? u / 12 : 0;
    const int comp = live ? (int)(u - t * 12) : 0;
    double *bufA = sm + (size_t)(threadIdx.x / tpi) * 2 * stride, *bufB = bufA + stride;
    int l4[4], dims[4], ns[4];
    for (int k = 0; k < 4; ++k) {
        l4[k] = live ? lsh[rows[5 * t + k]] : 0;
        dims[k] = dv_ncart(l4[k]);
        ns[k] = dv_nsph(l4[k]);
    }
    const int ncar = dims[0] * dims[1] * dims[2] * dims[3];
    const int nsp = ns[0] * ns[1] * ns[2] * ns[3];
    if (live) {
        const double *src = cart + cart_off[t] + (int64_t)comp * ncar;
        for (int x = lane; x < ncar; x += tpi) bufA[x] = src[x];
    }
    __syncthreads();
    for (int pos = 0; pos < 4; ++pos) {
        int before = 1, after = 1;
        for (int k = 0; k < pos; ++k) before *= dims[k];
        for (int k = pos + 1; k < 4; ++k) after *= dims[k];
        const double *T = eri_sph_T[l4[pos]];
        const int nc = dims[pos], nsv = ns[pos];
        const double *in = (pos % 2 == 0) ? bufA : bufB;
        double *o = pos == 3 ? dst + (live ? dst_off[t] : 0) + (int64_t)comp * nsp : ((pos % 2 == 0) ? bufB : bufA);
        const int total = live ? before * nsv * after : 0;
        for (int x = lane; x < total; x += tpi) {
            const int y = x % after, rr = x / after, sv = rr % nsv, bb = rr / nsv;
            double acc = 0.0;
            for (int c = 0; c < nc; ++c) acc += T[sv * nc + c] * in[(bb * nc + c) * after + y];
            o[x] = acc;
        }
        dims[pos] = nsv;
        __syncthreads();
    }
}

// FP64 FMA issue rate: every lane runs eight independent chains of fused
// multiply-adds, eight waves per SIMD.
constexpr int FMA_CHAINS = 8, FMA_ITERS = 4096;

// The chains' sum is compared with `never` (a value it cannot take, passed at
// run time so that the compiler cannot drop the chains); only then is it
// stored, always to out[0], so the one-element sink is never written past.
__global__ void __launch_bounds__(256) k_fma_rate(double *out, double a, double b, double never)
{
    double v[FMA_CHAINS];
#pragma unroll
    for (int c = 0; c < FMA_CHAINS; ++c) v[c] = threadIdx.x + c;
    for (int i = 0; i < FMA_ITERS; ++i) {
#pragma unroll
        for (int c = 0; c < FMA_CHAINS; ++c) v[c] = fma(v[c], a, b);
    }
    double t = 0.0;
#pragma unroll
    for (int c = 0; c < FMA_CHAINS; ++c) t += v[c];
    if (t == never) out[0] = t;
}


inline unsigned nblk(int64_t n, int bs) { return (unsigned)((n + bs - 1) / bs); }

// ---------------------------------------------------------------------------
// caller workspace
// ---------------------------------------------------------------------------
// Every device buffer of a plan, and of a digestion or derivative call, is a
// slice of a workspace the caller allocated.  The same layout code runs twice:
// once without a base pointer, only adding up the bytes (the size query), and
// once carving the caller's workspace.
struct WsShort {
};

struct Arena {
    char *base = nullptr;
    size_t cap = 0, used = 0;
    Arena() = default;
    Arena(void *b, size_t c) : base((char *)b), cap(c) {}
    template <class T>
    T *take(size_t n)
    {
        const size_t at = (used + 255) / 256 * 256;
        used = at + (n ? n : 1) * sizeof(T);
        if (!base) return nullptr;
        if (used > cap) throw WsShort{};
        return reinterpret_cast<T *>(base + at);
    }
};

}  // namespace

// ---------------------------------------------------------------------------
// plan
// ---------------------------------------------------------------------------

struct EriBlock {
    int cid;
    int64_t start, count, out_off;
    int64_t n_k1;  // leading quartets with K_a K_b K_c K_d = 1
    int na, nb, nc, nd;  // functions per shell of the class (spherical or Cartesian)
};

// stream lanes: the caller's stream plus up to ERI_MAX_SIDE_STREAMS side streams
constexpr int ERI_LANES = ERI_MAX_SIDE_STREAMS + 1;

struct eri_plan {
    int flags = 0;
    bool sph = false;
    bool screened = false;
    int device = 0;
    int nshell = 0, nbf = 0;
    int64_t npairs = 0, nq = 0, nout = 0;
    double *d_cen = nullptr, *d_exps = nullptr, *d_cn = nullptr, *d_ppd = nullptr, *d_S = nullptr;
    int *d_l = nullptr, *d_nprim = nullptr, *d_off = nullptr, *d_bf = nullptr, *d_nfun = nullptr;
    int4 *d_pinfo = nullptr;
    // explicit quartet lists (plans built from a quartet list)
    int *d_qbra = nullptr, *d_qket = nullptr, *d_qmap = nullptr;
    int64_t *d_qsrc = nullptr;  // input position of the quartet in each slot
    double *d_boys = nullptr;
    double *d_scratch = nullptr;
    int scratch_wgs = 0;
    long long scratch_doubles = 0;  // per workgroup slice
    double *d_unfused = nullptr;    // work buffer of the unfused-spherical ablation build
    int grid_cap = 2048;            // persistent register-tier grid (8 workgroups per CU)
    std::vector<EriBlock> blocks;
    // screened plans: per (block, bra rank) the length of the surviving ket
    // prefix and its running offset; slot lists are expanded per chunk
    BlockDesc *d_bd = nullptr;
    int nbd = 0;
    int64_t nent = 0;
    int64_t *d_ent_off = nullptr;
    int *d_porder = nullptr, *d_pair_i = nullptr;
    int64_t chunk_q = 1 << 22;  // quartets per chunk
    int *d_chunk = nullptr;     // ERI_LANES x (bra list, ket list) x chunk_q
    size_t ws_used = 0;
    // host copies of the shells (derivative calls build their auxiliary shells from them)
    std::vector<int> hl, hk, hoff;
    std::vector<double> hcen, hexp, hcn;
    // side streams registered by the caller (eri_plan_set_streams)
    int nside = 0;
    hipStream_t side[ERI_MAX_SIDE_STREAMS] = {};
    hipEvent_t ev_fork = nullptr, ev_side[ERI_MAX_SIDE_STREAMS] = {};

    ~eri_plan()
    {
        if (ev_fork) {
            (void)hipEventDestroy(ev_fork);
            for (int i = 0; i < ERI_MAX_SIDE_STREAMS; ++i) (void)hipEventDestroy(ev_side[i]);
        }
    }
};

namespace {

template <class T>
void upload(T *dst, const T *src, size_t n, hipStream_t s)
{
    if (n) HIP_CHECK(hipMemcpyAsync(dst, src, n * sizeof(T), hipMemcpyHostToDevice, s));
}

// hipCUB primitives on caller temp storage; with tmp == nullptr they only
// report the temp bytes they need (no device work)
size_t scan_i64(const int64_t *in, int64_t *out, int64_t n, void *tmp, size_t bytes, hipStream_t s)
{
    if (n <= 0) return 0;
    if (!tmp) bytes = 0;
    HIP_CHECK(hipcub::DeviceScan::ExclusiveSum(tmp, bytes, in, out, (int)n, s));
    return bytes;
}

size_t scan_i32(const int *in, int *out, int64_t n, void *tmp, size_t bytes, hipStream_t s)
{
    if (n <= 0) return 0;
    if (!tmp) bytes = 0;
    HIP_CHECK(hipcub::DeviceScan::ExclusiveSum(tmp, bytes, in, out, (int)n, s));
    return bytes;
}

template <class V>
size_t sort_pairs_u64(uint64_t *keys_in, uint64_t *keys_out, V *v_in, V *v_out, int64_t n, void *tmp, size_t bytes,
                      hipStream_t s)
{
    if (n <= 0) return 0;
    if (!tmp) bytes = 0;
    HIP_CHECK(hipcub::DeviceRadixSort::SortPairs(tmp, bytes, keys_in, keys_out, v_in, v_out, (int)n, 0, 64, s));
    return bytes;
}

// output kind of the class kernels a plan launches (the unfused-spherical
// ablation build runs the Cartesian kernels for spherical plans)
inline bool kernel_sph(const eri_plan *P)
{
#ifdef ERI_UNFUSED_SPHERICAL
    return false;
#else
    return P->sph;
#endif
}

inline bool kernel_sph_flags(bool sph)
{
#ifdef ERI_UNFUSED_SPHERICAL
    (void)sph;
    return false;
#else
    return sph;
#endif
}

// memory-tier scratch doubles per workgroup the given classes need
long long scratch_need(const std::vector<int> &cids, bool ksph)
{
    long long need = 0;
    for (int cid : cids) {
        const EriClassEntry *ce = find_class(cid, ksph);
        if (ce && ce->tier == 'M') need = std::max(need, ce->scratch_doubles);
    }
    return need;
}

#ifdef ERI_UNFUSED_SPHERICAL
// work buffer of the unfused path (three Cartesian chunks, 800 MB: a few hundred
// (gg|gg) quartets per chunk, so that its class launches are not tiny), doubles
constexpr int64_t UNFUSED_DOUBLES = int64_t(3) << 25;
#endif

void launch_class_kind(const eri_plan *P, int cid, bool sph, const int *qbra, const int *qket, int64_t n, double *out,
                       hipStream_t s, int64_t n_k1, const int4 *pinfo = nullptr)
{
    const EriClassEntry *ce = find_class(cid, sph);
    if (!ce) {
        g_last_error = "no kernel for class " + std::to_string(cid);
        throw HipFail{hipErrorInvalidValue};
    }
    EriClassArgs a;
    a.qbra = qbra;
    a.qket = qket;
    a.pair_info = pinfo ? pinfo : P->d_pinfo;
    a.ppd = P->d_ppd;
    a.cen = P->d_cen;
    a.boys = P->d_boys;
    a.scratch = P->d_scratch;
    a.scratch_wgs = P->scratch_wgs;
    a.grid_cap = P->grid_cap;
    // an explicit plan's own lists pair slot s with pairs 2s and 2s + 1: kernels
    // may then skip reading them
    long long base = -1;
    if (!pinfo && !P->screened && qbra >= P->d_qbra && qbra < P->d_qbra + P->nq &&
        qket == P->d_qket + (qbra - P->d_qbra))
        base = 2 * (long long)(qbra - P->d_qbra);
    const int blk = nfun(ce->la, sph) * nfun(ce->lb, sph) * nfun(ce->lc, sph) * nfun(ce->ld, sph);
    if (ce->tier == 'M' && ce->scratch_doubles > 0 && (!P->d_scratch || P->scratch_doubles < ce->scratch_doubles)) {
        g_last_error = "memory-tier class without scratch";
        throw HipFail{hipErrorInvalidValue};
    }
    // the uncontracted prefix goes to the K4 = 1 kernel; large ranges are split so
    // that every grid stays within int range
    const int64_t CH = 1 << 26;
    for (int part = 0; part < 2; ++part) {
        const int64_t lo = part == 0 ? 0 : n_k1, hi = part == 0 ? n_k1 : n;
        for (int64_t b = lo; b < hi; b += CH) {
            const int64_t m = std::min(CH, hi - b);
            a.qbra = qbra + b;
            a.qket = qket + b;
            a.pair_base = base >= 0 ? base + 2 * b : -1;
            a.nq = (int)m;
            a.out = out + b * blk;
            (part == 0 ? ce->launch_k1 : ce->launch)(a, s);
            HIP_CHECK(hipGetLastError());
        }
    }
}

#ifdef ERI_UNFUSED_SPHERICAL
// Ablation build only (the "no spherical fusion" variant of section V-B of
// "FusionRCG"): a spherical block is computed as its Cartesian block, written
// out, and then transformed on all four indices, Eq. (17), instead of the
// stepwise fusion of Eq. (14).  One workgroup per quartet, four one-index
// passes through two work buffers (the plan's unfused work buffer: calls on
// one plan from several streams run one after another on the caller's stream).
__global__ void k_sph_unfused(int64_t n, int la, int lb, int lc, int ld, const double *cart, double *w0, double *w1,
                              double *dst)
{
    const int64_t t = blockIdx.x;
    if (t >= n) return;
    const int l4[4] = {la, lb, lc, ld};
    int dims[4], ns[4];
    for (int k = 0; k < 4; ++k) {
        dims[k] = (l4[k] + 1) * (l4[k] + 2) / 2;
        ns[k] = 2 * l4[k] + 1;
    }
    const int64_t ncar = (int64_t)dims[0] * dims[1] * dims[2] * dims[3];
    const int nsp = ns[0] * ns[1] * ns[2] * ns[3];
    const double *in = cart + t * ncar;
    for (int pos = 0; pos < 4; ++pos) {
        int before = 1, after = 1;
        for (int k = 0; k < pos; ++k) before *= dims[k];
        for (int k = pos + 1; k < 4; ++k) after *= dims[k];
        const double *T = eri_sph_T[l4[pos]];
        const int nc = dims[pos], nsv = ns[pos];
        double *o = pos == 3 ? dst + t * nsp : ((pos % 2 == 0) ? w0 : w1) + t * ncar;
        const int total = before * nsv * after;
        for (int x = threadIdx.x; x < total; x += blockDim.x) {
            const int y = x % after, rr = x / after, sv = rr % nsv, bb = rr / nsv;
            double acc = 0.0;
            for (int c = 0; c < nc; ++c) acc += T[sv * nc + c] * in[((int64_t)bb * nc + c) * after + y];
            o[x] = acc;
        }
        dims[pos] = nsv;
        in = o;
        __syncthreads();
    }
}

void launch_class(const eri_plan *P, int cid, const int *qbra, const int *qket, int64_t n, double *out, hipStream_t s,
                  int64_t n_k1 = 0, const int4 *pinfo = nullptr)
{
    if (!P->sph) {
        launch_class_kind(P, cid, false, qbra, qket, n, out, s, n_k1, pinfo);
        return;
    }
    const EriClassEntry *ce = find_class(cid, false);
    if (!ce) {
        g_last_error = "no kernel for class " + std::to_string(cid);
        throw HipFail{hipErrorInvalidValue};
    }
    const int64_t nc = (int64_t)ncart(ce->la) * ncart(ce->lb) * ncart(ce->lc) * ncart(ce->ld);
    const int64_t ns = (int64_t)nsph(ce->la) * nsph(ce->lb) * nsph(ce->lc) * nsph(ce->ld);
    const int64_t chunk = std::max<int64_t>(1, std::min<int64_t>(n, (UNFUSED_DOUBLES / 3) / nc));
    double *cart = P->d_unfused, *w0 = cart + chunk * nc, *w1 = w0 + chunk * nc;
    for (int64_t b = 0; b < n; b += chunk) {
        const int64_t m = std::min(chunk, n - b);
        const int64_t k1 = std::min(m, std::max<int64_t>(0, n_k1 - b));
        launch_class_kind(P, cid, false, qbra + b, qket + b, m, cart, s, k1, pinfo);
        hipLaunchKernelGGL(k_sph_unfused, dim3((unsigned)m), dim3(256), 0, s, m, ce->la, ce->lb, ce->lc, ce->ld, cart,
                           w0, w1, out + b * ns);
        HIP_CHECK(hipGetLastError());
    }
}
#else
void launch_class(const eri_plan *P, int cid, const int *qbra, const int *qket, int64_t n, double *out, hipStream_t s,
                  int64_t n_k1 = 0, const int4 *pinfo = nullptr)
{
    launch_class_kind(P, cid, P->sph, qbra, qket, n, out, s, n_k1, pinfo);
}
#endif

inline int *chunk_bra(const eri_plan *P, int lane) { return P->d_chunk + (size_t)lane * 2 * P->chunk_q; }
inline int *chunk_ket(const eri_plan *P, int lane) { return chunk_bra(P, lane) + P->chunk_q; }

// quartet lists of plan slots [s, s + m): the plan's own arrays, or for a
// screened plan the lane's chunk lists after expansion (m <= chunk_q)
void slot_lists(const eri_plan *P, int64_t s, int64_t m, const int **qb, const int **qk, hipStream_t st, int lane)
{
    if (!P->screened) {
        *qb = P->d_qbra + s;
        *qk = P->d_qket + s;
        return;
    }
    int *dqb = chunk_bra(P, lane), *dqk = chunk_ket(P, lane);
    hipLaunchKernelGGL(k_expand, dim3(nblk(m, 256)), dim3(256), 0, st, s, m, P->nent, P->d_ent_off, P->d_bd, P->nbd,
                       P->d_porder, P->d_pinfo, P->d_pair_i, dqb, dqk, (int *)nullptr);
    HIP_CHECK(hipGetLastError());
    *qb = dqb;
    *qk = dqk;
}

// Calls over several class blocks spread the blocks over the caller's stream
// and the side streams the caller registered, so that the last waves of one
// class kernel overlap the first waves of the next; the caller's stream then
// waits for the side streams.  Blocks of memory-tier classes that use the
// plan's scratch stay on the caller's stream, one after another.
int lanes_of(const eri_plan *P)
{
#ifdef ERI_UNFUSED_SPHERICAL
    (void)P;
    return 1;  // the unfused path shares one work buffer
#else
    return 1 + P->nside;
#endif
}

void side_fork(const eri_plan *P, hipStream_t s, int lanes)
{
    HIP_CHECK(hipEventRecord(P->ev_fork, s));
    for (int i = 0; i + 1 < lanes; ++i) HIP_CHECK(hipStreamWaitEvent(P->side[i], P->ev_fork, 0));
}

void side_join(const eri_plan *P, hipStream_t s, int lanes)
{
    for (int i = 0; i + 1 < lanes; ++i) {
        HIP_CHECK(hipEventRecord(P->ev_side[i], P->side[i]));
        HIP_CHECK(hipStreamWaitEvent(s, P->ev_side[i], 0));
    }
}

inline hipStream_t lane_stream(const eri_plan *P, int lane, hipStream_t s) { return lane == 0 ? s : P->side[lane - 1]; }

bool uses_scratch(const eri_plan *P, int cid)
{
    const EriClassEntry *ce = find_class(cid, kernel_sph(P));
    return ce && ce->tier == 'M' && ce->scratch_doubles > 0;
}

void compute_range(const eri_plan *P, const EriBlock &B, int64_t first, int64_t count, double *out, hipStream_t st,
                   int lane)
{
    const int64_t blk = (int64_t)B.na * B.nb * B.nc * B.nd;
    const int64_t step = P->screened ? P->chunk_q : std::max<int64_t>(count, 1);
    for (int64_t c = first; c < first + count; c += step) {
        const int64_t m = std::min(step, first + count - c);
        const int *qb = nullptr, *qk = nullptr;
        slot_lists(P, B.start + c, m, &qb, &qk, st, lane);
        const int64_t nk1 = std::max<int64_t>(0, std::min<int64_t>(B.n_k1 - c, m));
        launch_class(P, B.cid, qb, qk, m, out + (c - first) * blk, st, nk1);
    }
}

__global__ void k_add_mat(int n, const double *X, int ldx, double *Y, int ldy)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (int64_t)n * n) return;
    const int x = (int)(t / n), y = (int)(t - (int64_t)x * n);
    Y[(size_t)x * ldy + y] += X[(size_t)x * ldx + y];
}

// ---------------------------------------------------------------------------
// J and K digestion, chunk by chunk
// ---------------------------------------------------------------------------
// Integrals of the chunk, per-quartet contribution vectors, entries sorted by
// target (stable), then each target's run added in entry order.  The chunks
// are spread over stream lanes (the caller's stream and its registered side
// streams), each with its own chunk buffers and its own J and A accumulators,
// chunk i of the plan going to lane i mod (number of lanes) (chunks of
// memory-tier classes that use the plan's scratch all go to lane 0).  After
// the lanes join, lanes 1, 2, ... are added into lane 0's J and A in that
// order, so the sums are deterministic.
struct ChunkLane {
    double *ints = nullptr, *cb = nullptr, *kv = nullptr;  // integrals, J and K contribution vectors of a chunk
    double *J = nullptr, *A = nullptr;                     // lane accumulators (lane 0's J is the caller's)
    int *ek = nullptr, *ek2 = nullptr, *ruk = nullptr, *rlen = nullptr, *rst = nullptr, *nruns = nullptr;
    int *eo = nullptr, *eo2 = nullptr;  // entry offsets into the lane's contribution vectors
    void *tmp = nullptr;
    size_t tmp_bytes = 0;
};

// bits of the smallest radix that holds keys 0..maxkey
inline int key_bits(int64_t maxkey)
{
    int b = 1;
    while (b < 31 && (int64_t(1) << b) <= maxkey) ++b;
    return b;
}

struct DigestShape {
    int lanes;
    int64_t CQ, CO, CB, NE;
};

DigestShape digest_shape(const eri_plan *P, bool wantJ, bool wantK)
{
    DigestShape d;
    d.lanes = lanes_of(P);
    d.CQ = std::min<int64_t>(P->chunk_q, std::max<int64_t>(P->nq, 1));
    int64_t cbt = 0;
    for (const EriBlock &B : P->blocks) {
        const int64_t w = std::max<int64_t>(wantJ ? B.na * B.nb + B.nc * B.nd : 0,
                                            wantK ? B.na * B.nc + B.nb * B.nc + B.na * B.nd + B.nb * B.nd : 0);
        cbt += B.count * w;
    }
    const int64_t big = d.lanes > 1 ? 26 : 27;
    d.CO = std::min<int64_t>(int64_t(1) << big, std::max<int64_t>(P->nout, 1));
    d.CB = std::min<int64_t>(int64_t(1) << (big - 1), std::max<int64_t>(cbt, 1024));
    d.NE = (wantK ? 4 : 2) * d.CQ;
    return d;
}

void digest_layout(Arena &A, const eri_plan *P, bool wantJ, bool wantK, const DigestShape &d, std::vector<ChunkLane> &L,
                   double **kacc)
{
    const int n = P->nbf;
    L.assign(d.lanes, ChunkLane());
    size_t t1 = 0, t2 = 0, t3 = 0;
    const int n2 = (int)d.NE;
    HIP_CHECK(hipcub::DeviceRadixSort::SortPairs(nullptr, t1, (int *)nullptr, (int *)nullptr, (int *)nullptr,
                                                 (int *)nullptr, n2, 0, 32));
    HIP_CHECK(hipcub::DeviceRunLengthEncode::Encode(nullptr, t2, (int *)nullptr, (int *)nullptr, (int *)nullptr,
                                                    (int *)nullptr, n2));
    HIP_CHECK(hipcub::DeviceScan::ExclusiveSum(nullptr, t3, (int *)nullptr, (int *)nullptr, n2));
    const size_t tb = std::max(t1, std::max(t2, t3));
    for (int l = 0; l < d.lanes; ++l) {
        ChunkLane &W = L[l];
        W.ints = A.take<double>(d.CO);
        if (wantJ) W.cb = A.take<double>(d.CB);
        if (wantK) W.kv = A.take<double>(d.CB);
        W.ek = A.take<int>(d.NE);
        W.ek2 = A.take<int>(d.NE);
        W.eo = A.take<int>(d.NE);
        W.eo2 = A.take<int>(d.NE);
        W.ruk = A.take<int>(d.NE);
        W.rlen = A.take<int>(d.NE);
        W.rst = A.take<int>(d.NE);
        W.nruns = A.take<int>(1);
        W.tmp = A.take<char>(tb);
        W.tmp_bytes = tb;
        if (wantJ && l > 0) W.J = A.take<double>((size_t)n * n);
        if (wantK) W.A = A.take<double>((size_t)n * n);
    }
    *kacc = wantK ? L[0].A : nullptr;
}

// One stream lane, chunk buffers halved until the layout fits in `cap` bytes
// (at least one quartet of the largest class block per chunk).  Returns false
// if even that does not fit.
bool digest_shape_capped(const eri_plan *P, bool wantJ, bool wantK, size_t cap, DigestShape &d)
{
    d = digest_shape(P, wantJ, wantK);
    d.lanes = 1;
    int64_t blk_max = 1;
    for (const EriBlock &B : P->blocks) blk_max = std::max<int64_t>(blk_max, (int64_t)B.na * B.nb * B.nc * B.nd);
    for (;;) {
        Arena count;
        std::vector<ChunkLane> L;
        double *kacc = nullptr;
        digest_layout(count, P, wantJ, wantK, d, L, &kacc);
        if (count.used <= cap) return true;
        if (d.CO <= blk_max && d.CB <= 1024 && d.CQ <= 1) return false;
        d.CO = std::max<int64_t>(blk_max, d.CO / 2);
        d.CB = std::max<int64_t>(1024, d.CB / 2);
        d.CQ = std::max<int64_t>(1, d.CQ / 2);
        d.NE = (wantK ? 4 : 2) * d.CQ;
    }
}

// Quartet ranges to digest: every block whole, or slots [first, first + count)
// of one block.
struct DigestRange {
    int block = -1;  // -1: all blocks
    int64_t first = 0, count = 0;
};

// accumulate: J gets the range's contributions added to what it holds instead
// of being overwritten.
void digest_JK_run(const eri_plan *P, const double *D, int ldd, double *J, int ldj, double *K, int ldk, Arena &ws,
                   hipStream_t s, const DigestShape *shape = nullptr, DigestRange rg = DigestRange(),
                   bool accumulate = false)
{
    const int b0 = rg.block < 0 ? 0 : rg.block, b1 = rg.block < 0 ? (int)P->blocks.size() : rg.block + 1;
    const DigestShape d = shape ? *shape : digest_shape(P, J != nullptr, K != nullptr);
    std::vector<ChunkLane> L;
    double *kacc = nullptr;
    digest_layout(ws, P, J != nullptr, K != nullptr, d, L, &kacc);
    const int NL = d.lanes;
    const int n = P->nbf;
    if (NL > 1) side_fork(P, s, NL);
    for (int l = 0; l < NL; ++l) {
        const hipStream_t ls = lane_stream(P, l, s);
        ChunkLane &W = L[l];
        double *Jl = l == 0 ? J : W.J;
        const int ldl = l == 0 ? ldj : n;
        if (J && !(accumulate && l == 0))
            hipLaunchKernelGGL(k_zero_mat, dim3(nblk((int64_t)n * n, 256)), dim3(256), 0, ls, n, Jl, ldl);
        if (K) hipLaunchKernelGGL(k_zero_mat, dim3(nblk((int64_t)n * n, 256)), dim3(256), 0, ls, n, W.A, n);
        HIP_CHECK(hipGetLastError());
    }
    // J entries of consecutive chunks of a lane collect in its buffers and are
    // sorted and added together when the next chunk would not fit (and at the
    // end): fewer, larger sorts.  The flush points follow from the plan and the
    // shape alone, and the sort is stable, so every sum keeps a fixed order.
    struct Pending {
        int64_t e = 0, cb = 0;
    };
    std::vector<Pending> pend(NL);
    auto sort_runs = [&](ChunkLane &W, hipStream_t ls, int n2, int bits) {
        size_t tb = W.tmp_bytes;
        HIP_CHECK(hipcub::DeviceRadixSort::SortPairs(W.tmp, tb, W.ek, W.ek2, W.eo, W.eo2, n2, 0, bits, ls));
        tb = W.tmp_bytes;
        HIP_CHECK(hipcub::DeviceRunLengthEncode::Encode(W.tmp, tb, W.ek2, W.ruk, W.rlen, W.nruns, n2, ls));
        tb = W.tmp_bytes;
        HIP_CHECK(hipcub::DeviceScan::ExclusiveSum(W.tmp, tb, W.rlen, W.rst, n2, ls));
    };
    auto flush_J = [&](int l) {
        if (pend[l].e == 0) return;
        const hipStream_t ls = lane_stream(P, l, s);
        ChunkLane &W = L[l];
        sort_runs(W, ls, (int)pend[l].e, key_bits(P->npairs));
        // at most one run per pair key (and one for the sentinel key); workgroups
        // past the device-side run count exit at once
        const int64_t nrun = std::min<int64_t>(pend[l].e, P->npairs + 1);
        hipLaunchKernelGGL(k_add_runs, dim3((unsigned)nrun), dim3(RUN_THREADS), 0, ls, W.nruns, W.ruk, W.rst,
                           W.rlen, W.eo2, W.cb, P->d_pinfo, P->d_bf, P->d_nfun, (int)P->npairs,
                           l == 0 ? J : W.J, l == 0 ? ldj : n);
        HIP_CHECK(hipGetLastError());
        pend[l] = Pending();
    };
    int64_t chunk_index = 0;
    for (int bi = b0; bi < b1; ++bi) {
        const EriBlock &B = P->blocks[bi];
        const int nab = B.na * B.nb, ncd = B.nc * B.nd;
        const int nkv = B.na * B.nc + B.nb * B.nc + B.na * B.nd + B.nb * B.nd;
        const int64_t blk = (int64_t)nab * ncd;
        int64_t step = std::min(d.CQ, d.CO / blk);
        if (J) step = std::min<int64_t>(step, d.CB / (nab + ncd));
        if (K) step = std::min<int64_t>(step, d.CB / nkv);
        step = std::max<int64_t>(1, step);
        const bool scratch_class = uses_scratch(P, B.cid);
        const int64_t c0 = rg.block < 0 ? 0 : rg.first, c1 = rg.block < 0 ? B.count : rg.first + rg.count;
        for (int64_t c = c0; c < c1; c += step, ++chunk_index) {
            const int l = scratch_class ? 0 : (int)(chunk_index % NL);
            const hipStream_t ls = lane_stream(P, l, s);
            ChunkLane &W = L[l];
            const int64_t m = std::min(step, c1 - c);
            const int *qb = nullptr, *qk = nullptr;
            slot_lists(P, B.start + c, m, &qb, &qk, ls, l);
            const int64_t nk1 = std::max<int64_t>(0, std::min<int64_t>(B.n_k1 - c, m));
            launch_class(P, B.cid, qb, qk, m, W.ints, ls, nk1);
            if (J) {
                const int64_t nv = m * (nab + ncd);
                if (pend[l].e + 2 * m > d.NE || pend[l].cb + nv > d.CB) flush_J(l);
                hipLaunchKernelGGL(k_digest_rows, dim3((unsigned)nblk(nv, 256)), dim3(256), 0, ls, nv, B.na, B.nb,
                                   B.nc, B.nd, qb, qk, P->d_pinfo, P->d_bf, W.ints, D, ldd, W.cb + pend[l].cb);
                hipLaunchKernelGGL(k_chunk_entries, dim3(nblk(m, 256)), dim3(256), 0, ls, (int)m, qb, qk, nab, ncd,
                                   (int)P->npairs, pend[l].cb, W.ek + pend[l].e, W.eo + pend[l].e);
                HIP_CHECK(hipGetLastError());
                pend[l].e += 2 * m;
                pend[l].cb += nv;
                if (K) flush_J(l);  // the K entries below reuse the entry buffers
            }
            if (K) {
                const int64_t nkt = m * nkv;
                hipLaunchKernelGGL(k_kdigest_rows, dim3((unsigned)nblk(nkt, 256)), dim3(256), 0, ls, nkt, B.na, B.nb,
                                   B.nc, B.nd, qb, qk, P->d_pinfo, P->d_bf, W.ints, D, ldd, W.kv);
                hipLaunchKernelGGL(k_kchunk_entries, dim3(nblk(m, 256)), dim3(256), 0, ls, (int)m, qb, qk, P->d_pinfo,
                                   P->nshell, B.na, B.nb, B.nc, B.nd, W.ek, W.eo);
                HIP_CHECK(hipGetLastError());
                sort_runs(W, ls, (int)(4 * m), key_bits((int64_t)P->nshell * P->nshell));
                // at most one run per target block key (and one for the sentinel key)
                const int64_t nrun = std::min<int64_t>(4 * m, (int64_t)P->nshell * P->nshell + 1);
                hipLaunchKernelGGL(k_add_runs_K, dim3((unsigned)nrun), dim3(RUN_THREADS), 0, ls, W.nruns, W.ruk,
                                   W.rst, W.rlen, W.eo2, W.kv, P->nshell, P->d_bf, P->d_nfun, W.A, n);
                HIP_CHECK(hipGetLastError());
            }
        }
    }
    if (J)
        for (int l = 0; l < NL; ++l) flush_J(l);
    if (NL > 1) side_join(P, s, NL);
    for (int l = 1; l < NL; ++l) {
        if (J)
            hipLaunchKernelGGL(k_add_mat, dim3(nblk((int64_t)n * n, 256)), dim3(256), 0, s, n, L[l].J, n, J, ldj);
        if (K)
            hipLaunchKernelGGL(k_add_mat, dim3(nblk((int64_t)n * n, 256)), dim3(256), 0, s, n, L[l].A, n, kacc, n);
        HIP_CHECK(hipGetLastError());
    }
    if (K) {
        hipLaunchKernelGGL(k_sym_add, dim3(nblk((int64_t)n * n, 256)), dim3(256), 0, s, n, kacc, n, K, ldk);
        HIP_CHECK(hipGetLastError());
    }
}

// ---------------------------------------------------------------------------
// plan build
// ---------------------------------------------------------------------------

// What the host knows before any device work: every buffer size.
struct BuildHost {
    int ns = 0, npr = 0;
    int64_t nq = 0;        // explicit lists
    int64_t np = 0;        // shell pairs
    int64_t nppd = 0;      // primitive pairs
    int64_t nent = 0;      // screened: (block, bra rank) entries
    int nbuck = 0, nbd = 0;
    size_t diag_doubles = 0;
    int64_t diag_q = 0;     // screened: sub-pair quartets per Schwarz batch
    int64_t nsub = 0;       // screened: sub-pairs of all pairs
    long long scratch = 0;
    int64_t chunk_q = 0;
    size_t cub = 0;
    std::vector<int> hbf, hnf;
    std::vector<int> kept;  // screened: kept primitive pairs of pair p = i(i+1)/2 + j
};

struct BuildBufs {
    double *raw = nullptr;
    // explicit
    int *q = nullptr;
    uint64_t *k0 = nullptr, *k1 = nullptr;
    int64_t *p0 = nullptr, *st = nullptr, *k1e = nullptr;
    // both
    int *w = nullptr, *z = nullptr;
    void *cub = nullptr;
    // screened
    uint64_t *pck = nullptr, *pck2 = nullptr, *ka = nullptr, *kb = nullptr, *bkey = nullptr;
    int *pidx = nullptr, *pidx2 = nullptr, *seq = nullptr, *o1 = nullptr, *head = nullptr, *hscan = nullptr,
        *bstart = nullptr;
    double *diag = nullptr;
    int64_t *cnt = nullptr, *idx = nullptr, *bs = nullptr;
    int4 *sub = nullptr;                 // sub-pairs of the Schwarz diagonals
    int64_t *kpo = nullptr, *boff = nullptr;
    int *dq = nullptr, *ksub = nullptr;  // sub-pair quartet lists of a batch; sub-pairs per pair
};

constexpr size_t DIAG_DOUBLES = size_t(1) << 24;  // Schwarz diagonal blocks per launch

void host_common(const eri_shells *sh, bool sph, BuildHost &H)
{
    H.ns = sh->nshell;
    H.npr = sh->prim_off[H.ns];
    H.hbf.assign(H.ns + 1, 0);
    H.hnf.assign(H.ns, 0);
    for (int i = 0; i < H.ns; ++i) {
        H.hnf[i] = nfun(sh->l[i], sph);
        H.hbf[i + 1] = H.hbf[i] + H.hnf[i];
    }
}

// canonical class id of a quartet of shells with angular momenta l4
int class_of(int li, int lj, int lk, int ll)
{
    const int pb = pair_class(std::max(li, lj), std::min(li, lj));
    const int pk = pair_class(std::max(lk, ll), std::min(lk, ll));
    return class_id_of(std::max(pb, pk), std::min(pb, pk));
}

// sizes of an explicit plan from its quartet count, the sum of its pairs'
// primitive pair counts and the classes present
void host_explicit_counts(const eri_shells *sh, int flags, int64_t nq, int64_t nppd, const bool *present,
                          BuildHost &H)
{
    host_common(sh, (flags & ERI_SPHERICAL) != 0, H);
    H.nq = nq;
    H.np = 2 * nq;
    H.nppd = nppd;
    std::vector<int> cids;
    for (int c = 0; c < ERI_NCLASS; ++c)
        if (present[c]) cids.push_back(c);
    H.scratch = scratch_need(cids, kernel_sph_flags((flags & ERI_SPHERICAL) != 0));
    H.cub = std::max(sort_pairs_u64<int64_t>(nullptr, nullptr, nullptr, nullptr, nq, nullptr, 0, nullptr),
                     scan_i32(nullptr, nullptr, H.np, nullptr, 0, nullptr));
}

void host_explicit(const eri_shells *sh, int flags, const int32_t *quartets, int64_t nq, BuildHost &H)
{
    int64_t nppd = 0;
    bool present[ERI_NCLASS] = {};
    for (int64_t x = 0; x < nq; ++x) {
        const int *q = quartets + 4 * x;
        nppd += (int64_t)sh->nprim[q[0]] * sh->nprim[q[1]] + (int64_t)sh->nprim[q[2]] * sh->nprim[q[3]];
        present[class_of(sh->l[q[0]], sh->l[q[1]], sh->l[q[2]], sh->l[q[3]])] = true;
    }
    host_explicit_counts(sh, flags, nq, nppd, present, H);
}

void host_screened(const eri_shells *sh, int flags, int64_t chunk_q, BuildHost &H)
{
    host_common(sh, (flags & ERI_SPHERICAL) != 0, H);
    const int ns = H.ns;
    H.np = (int64_t)ns * (ns + 1) / 2;
    std::vector<uint64_t> keys;
    keys.reserve(H.np);
    bool pc_present[15] = {};
    int64_t pc_count[15] = {}, pc_k2[15] = {}, pc_kmax2[15] = {};
    for (int i = 0; i < ns; ++i)
        for (int j = 0; j <= i; ++j) {
            const int a = sh->l[i] >= sh->l[j] ? i : j, b = a == i ? j : i;
            const int pc = pair_class(sh->l[a], sh->l[b]);
            const int64_t K = prim_pairs_kept(sh->centers, sh->prim_off, sh->exps, a, b);
            H.kept.push_back((int)K);
            H.nppd += K;
            const int64_t ks = (K + SCHWARZ_SUBK - 1) / SCHWARZ_SUBK;  // sub-pairs of the Schwarz diagonal
            H.nsub += ks;
            pc_k2[pc] += ks * ks;
            pc_kmax2[pc] = std::max(pc_kmax2[pc], ks * ks);
            keys.push_back(((uint64_t)pc << 16) | (uint64_t)K);
            pc_present[pc] = true;
            ++pc_count[pc];
        }
    if (H.nsub > (int64_t)INT32_MAX) {  // sub-pair indices of the Schwarz diagonals are 32-bit
        g_last_error = "too many Schwarz sub-pairs";
        throw HipFail{hipErrorInvalidValue};
    }
    std::sort(keys.begin(), keys.end());
    std::vector<int64_t> nB;
    for (size_t x = 0; x < keys.size(); ++x)
        if (x == 0 || keys[x] != keys[x - 1]) nB.push_back(1);
        else ++nB.back();
    H.nbuck = (int)nB.size();
    H.nbd = H.nbuck * (H.nbuck + 1) / 2;
    for (int B = 0; B < H.nbuck; ++B) H.nent += (int64_t)(B + 1) * nB[B];
    std::vector<int> cids;
    for (int pb = 0; pb < 15; ++pb)
        for (int pk = 0; pk <= pb; ++pk)
            if (pc_present[pb] && pc_present[pk]) cids.push_back(class_id_of(pb, pk));
    const bool sph = (flags & ERI_SPHERICAL) != 0;
    H.scratch = scratch_need(cids, kernel_sph_flags(sph));
    for (int pc = 0; pc < 15; ++pc) {
        if (!pc_count[pc]) continue;
        int la = 0;
        while ((la + 1) * (la + 2) / 2 <= pc) ++la;
        const size_t nab = (size_t)nfun(la, sph) * nfun(pc - la * (la + 1) / 2, sph);
        // a batch of the class's sub-pair quartets; at least every sub-pair quartet of its largest pair
        const size_t fit = std::max<size_t>(DIAG_DOUBLES / (nab * nab), (size_t)pc_kmax2[pc]);
        H.diag_doubles = std::max(H.diag_doubles, std::min<size_t>(fit, (size_t)pc_k2[pc]) * nab * nab);
        H.diag_q = std::max<int64_t>(H.diag_q, (int64_t)std::min<size_t>(fit, (size_t)pc_k2[pc]));
    }
    const int64_t nuq = H.np * (H.np + 1) / 2;
    H.chunk_q = std::min<int64_t>(chunk_q, std::max<int64_t>(nuq, 1));
    size_t c = sort_pairs_u64<int>(nullptr, nullptr, nullptr, nullptr, H.np, nullptr, 0, nullptr);
    c = std::max(c, scan_i32(nullptr, nullptr, H.np, nullptr, 0, nullptr));
    c = std::max(c, scan_i64(nullptr, nullptr, H.nent, nullptr, 0, nullptr));
    H.cub = c;
}

// Carve every buffer of a plan (and of its build) out of the arena.
void plan_layout(Arena &A, eri_plan *P, const BuildHost &H, BuildBufs &X)
{
    const int ns = H.ns;
    P->d_cen = A.take<double>((size_t)3 * ns);
    P->d_l = A.take<int>(ns);
    P->d_nprim = A.take<int>(ns);
    P->d_off = A.take<int>(ns + 1);
    P->d_bf = A.take<int>(ns + 1);
    P->d_nfun = A.take<int>(ns);
    P->d_exps = A.take<double>(H.npr);
    X.raw = A.take<double>(H.npr);
    P->d_cn = A.take<double>(H.npr);
    P->d_pinfo = A.take<int4>(H.np);
    X.w = A.take<int>(H.np + 1);
    X.z = A.take<int>(H.np + 1);
    P->d_ppd = A.take<double>((size_t)H.nppd * ERI_PP_STRIDE);
    X.cub = A.take<char>(H.cub);
    if (!P->screened) {
        const int64_t nq = H.nq;
        X.q = A.take<int>((size_t)4 * nq);
        X.k0 = A.take<uint64_t>(nq);
        X.k1 = A.take<uint64_t>(nq);
        X.p0 = A.take<int64_t>(nq);
        P->d_qsrc = A.take<int64_t>(nq);
        P->d_qmap = A.take<int>((size_t)5 * nq);
        P->d_qbra = A.take<int>(nq);
        P->d_qket = A.take<int>(nq);
        X.st = A.take<int64_t>(ERI_NCLASS + 1);
        X.k1e = A.take<int64_t>(ERI_NCLASS + 1);
    } else {
        const int64_t np = H.np;
        X.pck = A.take<uint64_t>(np);
        X.pck2 = A.take<uint64_t>(np);
        X.pidx = A.take<int>(np);
        X.pidx2 = A.take<int>(np);
        P->d_S = A.take<double>(np);
        X.diag = A.take<double>(H.diag_doubles);
        X.sub = A.take<int4>(H.nsub);
        X.kpo = A.take<int64_t>(np);
        X.boff = A.take<int64_t>(np);
        X.ksub = A.take<int>(np);
        X.dq = A.take<int>((size_t)2 * H.diag_q);
        X.seq = A.take<int>(np);
        X.ka = A.take<uint64_t>(np);
        X.kb = A.take<uint64_t>(np);
        X.o1 = A.take<int>(np);
        P->d_porder = A.take<int>(np);
        X.head = A.take<int>(np);
        X.hscan = A.take<int>(np);
        X.bstart = A.take<int>(H.nbuck + 1);
        X.bkey = A.take<uint64_t>(H.nbuck);
        P->d_bd = A.take<BlockDesc>(H.nbd);
        X.cnt = A.take<int64_t>(H.nent + 1);
        P->d_ent_off = A.take<int64_t>(H.nent + 1);
        P->d_pair_i = A.take<int>(np);
        X.idx = A.take<int64_t>(H.nbd + 1);
        X.bs = A.take<int64_t>(H.nbd + 1);
        P->chunk_q = H.chunk_q;
        P->d_chunk = A.take<int>((size_t)ERI_LANES * 2 * H.chunk_q);
    }
    if (H.scratch > 0) {
        P->d_scratch = A.take<double>((size_t)H.scratch * ERI_MEM_WGS);
        P->scratch_wgs = ERI_MEM_WGS;
        P->scratch_doubles = H.scratch;
    }
#ifdef ERI_UNFUSED_SPHERICAL
    if (P->sph) P->d_unfused = A.take<double>(UNFUSED_DOUBLES);
#endif
}

void make_pair_data(eri_plan *P, const BuildHost &H, BuildBufs &X, hipStream_t s)
{
    const int np = (int)P->npairs;
    if (np == 0) return;
    hipLaunchKernelGGL(k_copy_w, dim3(nblk(np, 256)), dim3(256), 0, s, np, P->d_pinfo, X.w);
    HIP_CHECK(hipGetLastError());
    scan_i32(X.w, X.z, np, X.cub, H.cub, s);
    hipLaunchKernelGGL(k_set_z, dim3(nblk(np, 256)), dim3(256), 0, s, np, P->d_pinfo, X.z);
    hipLaunchKernelGGL(k_pair_data, dim3(nblk(np, 128)), dim3(128), 0, s, np, P->d_pinfo, P->d_cen, P->d_off,
                       P->d_exps, P->d_cn, P->screened ? 1 : 0, P->d_ppd);
    HIP_CHECK(hipGetLastError());
}

void build_explicit(eri_plan *P, const BuildHost &H, BuildBufs &X, const int32_t *quartets, hipStream_t s)
{
    const int64_t nq = H.nq;
    P->nq = nq;
    P->npairs = 2 * nq;
    if (nq == 0) return;
    upload(X.q, quartets, (size_t)4 * nq, s);
    hipLaunchKernelGGL(k_explicit_keys, dim3(nblk(nq, 256)), dim3(256), 0, s, nq, X.q, P->d_l, P->d_nprim, X.k0, X.p0);
    HIP_CHECK(hipGetLastError());
    sort_pairs_u64(X.k0, X.k1, X.p0, P->d_qsrc, nq, X.cub, H.cub, s);
    hipLaunchKernelGGL(k_explicit_fill, dim3(nblk(nq, 256)), dim3(256), 0, s, nq, P->d_qsrc, X.q, P->d_l, P->d_nprim,
                       P->d_qmap, P->d_qbra, P->d_qket, P->d_pinfo);
    HIP_CHECK(hipGetLastError());
    const int NC = ERI_NCLASS;
    hipLaunchKernelGGL(k_class_starts, dim3(nblk(NC + 1, 128)), dim3(128), 0, s, nq, X.k1, X.st, X.k1e, NC);
    HIP_CHECK(hipGetLastError());
    std::vector<int64_t> st(NC + 1), k1e(NC + 1);
    HIP_CHECK(hipMemcpyAsync(st.data(), X.st, sizeof(int64_t) * (NC + 1), hipMemcpyDeviceToHost, s));
    HIP_CHECK(hipMemcpyAsync(k1e.data(), X.k1e, sizeof(int64_t) * (NC + 1), hipMemcpyDeviceToHost, s));
    make_pair_data(P, H, X, s);
    HIP_CHECK(hipStreamSynchronize(s));
    st[NC] = nq;
    int64_t out = 0;
    for (int c = 0; c < NC; ++c) {
        const int64_t cnt = st[c + 1] - st[c];
        if (cnt <= 0) continue;
        const EriClassEntry *ce = find_class(c, P->sph);
        if (!ce) {
            g_last_error = "class " + std::to_string(c) + " not built";
            throw HipFail{hipErrorInvalidValue};
        }
        EriBlock b{c, st[c], cnt, out, std::min(k1e[c], st[c + 1]) - st[c], nfun(ce->la, P->sph),
                   nfun(ce->lb, P->sph), nfun(ce->lc, P->sph), nfun(ce->ld, P->sph)};
        out += cnt * (int64_t)b.na * b.nb * b.nc * b.nd;
        P->blocks.push_back(b);
    }
    P->nout = out;
}

void build_screened(eri_plan *P, const BuildHost &H, BuildBufs &X, double tau, hipStream_t s)
{
    const int ns = P->nshell;
    const int64_t np = H.np;
    if (np > (int64_t)INT32_MAX / 2) {
        g_last_error = "too many shell pairs";
        throw HipFail{hipErrorInvalidValue};
    }
    P->npairs = np;
    // the host's kept counts, so that buckets and record offsets follow the sizes it reserved
    upload(X.w, H.kept.data(), (size_t)np, s);
    hipLaunchKernelGGL(k_all_pairs, dim3(nblk(np, 256)), dim3(256), 0, s, ns, P->d_l, X.w, P->d_pinfo, X.pck,
                       X.pidx);
    HIP_CHECK(hipGetLastError());
    make_pair_data(P, H, X, s);

    // --- Schwarz factors from the diagonal quartets (p|p), grouped by pair class,
    // each computed as the sum over its sub-pair quartets (k_sub_pairs)
    std::vector<int64_t> kpo(np);
    {
        int64_t o = 0;
        for (int64_t p = 0; p < np; ++p) {
            kpo[p] = o;
            o += (H.kept[p] + SCHWARZ_SUBK - 1) / SCHWARZ_SUBK;
        }
    }
    upload(X.kpo, kpo.data(), (size_t)np, s);
    hipLaunchKernelGGL(k_sub_pairs, dim3(nblk(np, 256)), dim3(256), 0, s, (int)np, P->d_pinfo, X.kpo, X.sub);
    HIP_CHECK(hipGetLastError());
    sort_pairs_u64(X.pck, X.pck2, X.pidx, X.pidx2, np, X.cub, H.cub, s);  // pidx2: pairs ordered by pair class
    std::vector<uint64_t> hpc(np);
    std::vector<int> hpidx(np);
    HIP_CHECK(hipMemcpyAsync(hpc.data(), X.pck2, sizeof(uint64_t) * np, hipMemcpyDeviceToHost, s));
    HIP_CHECK(hipMemcpyAsync(hpidx.data(), X.pidx2, sizeof(int) * np, hipMemcpyDeviceToHost, s));
    HIP_CHECK(hipStreamSynchronize(s));
    {
        std::vector<int> qb, qk, hk;
        std::vector<int64_t> hoff;
        int64_t i = 0;
        while (i < np) {
            int64_t j = i;
            while (j < np && hpc[j] == hpc[i]) ++j;
            const int pc = (int)hpc[i];
            int la = 0;
            while ((la + 1) * (la + 2) / 2 <= pc) ++la;
            const int lb = pc - la * (la + 1) / 2;
            const int64_t nab = nfun(la, P->sph) * nfun(lb, P->sph);
            const int64_t capb = std::min<int64_t>((int64_t)H.diag_doubles / (nab * nab), H.diag_q);
            for (int64_t t = i; t < j;) {
                qb.clear();
                qk.clear();
                hk.clear();
                hoff.clear();
                int64_t u = t, nb = 0;
                while (u < j) {
                    const int p = hpidx[u];
                    const int64_t k = (H.kept[p] + SCHWARZ_SUBK - 1) / SCHWARZ_SUBK;
                    if (nb + k * k > capb) break;
                    hoff.push_back(nb);
                    hk.push_back((int)k);
                    for (int64_t x = 0; x < k; ++x)
                        for (int64_t y = 0; y < k; ++y) {
                            qb.push_back((int)(kpo[p] + x));
                            qk.push_back((int)(kpo[p] + y));
                        }
                    nb += k * k;
                    ++u;
                }
                if (u == t) {  // cannot happen: capb holds the largest pair's sub-pair quartets
                    g_last_error = "Schwarz batch too small";
                    throw HipFail{hipErrorInvalidValue};
                }
                upload(X.dq, qb.data(), qb.size(), s);
                upload(X.dq + H.diag_q, qk.data(), qk.size(), s);
                upload(X.ksub, hk.data(), hk.size(), s);
                upload(X.boff, hoff.data(), hoff.size(), s);
                launch_class(P, class_id_of(pc, pc), X.dq, X.dq + H.diag_q, nb, X.diag, s, 0, X.sub);
                hipLaunchKernelGGL(k_schwarz_sum_max, dim3(nblk(u - t, 256)), dim3(256), 0, s, (int)(u - t),
                                   X.pidx2 + t, X.ksub, X.boff, X.diag, (int)nab, P->d_S);
                HIP_CHECK(hipGetLastError());
                t = u;
            }
            i = j;
        }
    }

    // --- bucket the pairs by (pair class, K_pair), rank by S descending (ties: pair index)
    {
        std::vector<int> h(np);
        for (int64_t p = 0; p < np; ++p) h[p] = (int)p;
        upload(X.seq, h.data(), np, s);
        hipLaunchKernelGGL(k_desc_keys, dim3(nblk(np, 256)), dim3(256), 0, s, (int)np, X.seq, P->d_S, X.ka);
        sort_pairs_u64(X.ka, X.kb, X.seq, X.o1, np, X.cub, H.cub, s);  // by S descending, stable: ties keep pair order
        HIP_CHECK(hipStreamSynchronize(s));                              // h is read by the upload above
    }
    hipLaunchKernelGGL(k_bucket_keys, dim3(nblk(np, 256)), dim3(256), 0, s, (int)np, X.o1, P->d_l, P->d_pinfo, X.ka);
    sort_pairs_u64(X.ka, X.kb, X.o1, P->d_porder, np, X.cub, H.cub, s);  // stable by bucket
    hipLaunchKernelGGL(k_heads, dim3(nblk(np, 256)), dim3(256), 0, s, (int)np, X.kb, X.head);
    scan_i32(X.head, X.hscan, np, X.cub, H.cub, s);
    int nb_last = 0, h_last = 0;
    HIP_CHECK(hipMemcpyAsync(&nb_last, X.hscan + np - 1, sizeof(int), hipMemcpyDeviceToHost, s));
    HIP_CHECK(hipMemcpyAsync(&h_last, X.head + np - 1, sizeof(int), hipMemcpyDeviceToHost, s));
    HIP_CHECK(hipStreamSynchronize(s));
    const int nbuck = nb_last + h_last;
    if (nbuck != H.nbuck) {
        g_last_error = "internal: bucket count differs from the host's";
        throw HipFail{hipErrorUnknown};
    }
    hipLaunchKernelGGL(k_bucket_table, dim3(nblk(np, 256)), dim3(256), 0, s, (int)np, X.kb, X.head, X.hscan, X.bstart,
                       X.bkey);
    std::vector<int> bstart(nbuck + 1);
    std::vector<uint64_t> bkey(nbuck);
    HIP_CHECK(hipMemcpyAsync(bstart.data(), X.bstart, sizeof(int) * nbuck, hipMemcpyDeviceToHost, s));
    HIP_CHECK(hipMemcpyAsync(bkey.data(), X.bkey, sizeof(uint64_t) * nbuck, hipMemcpyDeviceToHost, s));
    HIP_CHECK(hipStreamSynchronize(s));
    bstart[nbuck] = (int)np;

    // --- blocks (bra bucket >= ket bucket), ordered by (class, K_bra, K_ket)
    struct HB {
        int cid, kb, kk, B, Bk;
    };
    std::vector<HB> hb;
    for (int B = 0; B < nbuck; ++B)
        for (int Bk = 0; Bk <= B; ++Bk) {
            const int pcb = (int)(bkey[B] >> 16), pck = (int)(bkey[Bk] >> 16);
            hb.push_back({class_id_of(pcb, pck), (int)(bkey[B] & 0xffff), (int)(bkey[Bk] & 0xffff), B, Bk});
        }
    std::stable_sort(hb.begin(), hb.end(), [](const HB &x, const HB &y) {
        if (x.cid != y.cid) return x.cid < y.cid;
        if (x.kb != y.kb) return x.kb < y.kb;
        return x.kk < y.kk;
    });
    std::vector<BlockDesc> bd(hb.size());
    int64_t nent = 0;
    for (size_t i = 0; i < hb.size(); ++i) {
        const int B = hb[i].B, Bk = hb[i].Bk;
        bd[i] = BlockDesc{bstart[B], bstart[B + 1] - bstart[B], bstart[Bk], bstart[Bk + 1] - bstart[Bk], B == Bk ? 1 : 0,
                          nent};
        nent += bd[i].bra_n;
    }
    if (nent != H.nent || (int)bd.size() != H.nbd) {
        g_last_error = "internal: entry count differs from the host's";
        throw HipFail{hipErrorUnknown};
    }
    upload(P->d_bd, bd.data(), bd.size(), s);
    const double tau2 = tau * tau;
    if (nent) {
        hipLaunchKernelGGL(k_count, dim3(nblk(nent, 256)), dim3(256), 0, s, nent, P->d_bd, (int)bd.size(), P->d_porder,
                           P->d_S, tau2, X.cnt);
        HIP_CHECK(hipGetLastError());
        scan_i64(X.cnt, P->d_ent_off, nent, X.cub, H.cub, s);
    }
    int64_t lo = 0, lc = 0;
    if (nent) {
        HIP_CHECK(hipMemcpyAsync(&lo, P->d_ent_off + nent - 1, sizeof(int64_t), hipMemcpyDeviceToHost, s));
        HIP_CHECK(hipMemcpyAsync(&lc, X.cnt + nent - 1, sizeof(int64_t), hipMemcpyDeviceToHost, s));
        HIP_CHECK(hipStreamSynchronize(s));
    }
    const int64_t nq = lo + lc;
    P->nq = nq;
    hipLaunchKernelGGL(k_pair_hi, dim3(nblk(np, 256)), dim3(256), 0, s, (int)np, P->d_pinfo, P->d_pair_i);
    HIP_CHECK(hipGetLastError());
    P->nbd = (int)bd.size();
    P->nent = nent;
    // block starts -> class ranges
    std::vector<int64_t> hbase(bd.size());
    for (size_t i = 0; i < bd.size(); ++i) hbase[i] = bd[i].entry_base;
    std::vector<int64_t> bst(bd.size());
    if (!bd.empty() && nent) {
        // entry_base may equal nent for an empty trailing block: clamp, fix on host
        std::vector<int64_t> idx(bd.size());
        for (size_t i = 0; i < bd.size(); ++i) idx[i] = std::min<int64_t>(hbase[i], nent - 1);
        upload(X.idx, idx.data(), idx.size(), s);
        hipLaunchKernelGGL(k_gather_i64, dim3(nblk(bd.size(), 256)), dim3(256), 0, s, (int)bd.size(), P->d_ent_off,
                           X.idx, X.bs);
        HIP_CHECK(hipMemcpyAsync(bst.data(), X.bs, sizeof(int64_t) * bd.size(), hipMemcpyDeviceToHost, s));
        HIP_CHECK(hipStreamSynchronize(s));
        for (size_t i = 0; i < bd.size(); ++i)
            if (bd[i].bra_n == 0 || hbase[i] >= nent) bst[i] = nq;
    }
    int64_t outp = 0;
    size_t i = 0;
    while (i < hb.size()) {
        size_t j = i;
        while (j < hb.size() && hb[j].cid == hb[i].cid) ++j;
        const int64_t st = bst[i];
        const int64_t en = (j < hb.size()) ? bst[j] : nq;
        if (en > st) {
            const EriClassEntry *ce = find_class(hb[i].cid, P->sph);
            if (!ce) {
                g_last_error = "class " + std::to_string(hb[i].cid) + " not built";
                throw HipFail{hipErrorInvalidValue};
            }
            // the (K_bra = 1, K_ket = 1) bucket pair, when present, is the first of the class
            int64_t nk1 = 0;
            if (hb[i].kb == 1 && hb[i].kk == 1) nk1 = ((i + 1 < hb.size()) ? bst[i + 1] : nq) - bst[i];
            EriBlock b{hb[i].cid, st, en - st, outp, nk1, nfun(ce->la, P->sph), nfun(ce->lb, P->sph),
                       nfun(ce->lc, P->sph), nfun(ce->ld, P->sph)};
            outp += b.count * (int64_t)b.na * b.nb * b.nc * b.nd;
            P->blocks.push_back(b);
        }
        i = j;
    }
    P->nout = outp;
}

int translate(const HipFail &) { return ERI_E_HIP; }

int validate_shells(const eri_shells *sh)
{
    if (!sh || sh->nshell < 1 || !sh->centers || !sh->l || !sh->nprim || !sh->prim_off || !sh->exps || !sh->coefs)
        return ERI_E_INVALID;
    const int ns = sh->nshell;
    if (sh->prim_off[0] != 0) return ERI_E_INVALID;
    for (int s = 0; s < ns; ++s) {
        if (sh->l[s] < 0 || sh->l[s] > ERI_MAX_L) return ERI_E_INVALID;
        if (sh->nprim[s] < 1 || sh->nprim[s] > ERI_MAX_PRIM) return ERI_E_INVALID;
        if (sh->prim_off[s + 1] - sh->prim_off[s] != sh->nprim[s]) return ERI_E_INVALID;
        for (int c = 0; c < 3; ++c)
            if (!std::isfinite(sh->centers[3 * s + c])) return ERI_E_INVALID;
        for (int k = sh->prim_off[s]; k < sh->prim_off[s + 1]; ++k)
            if (!(sh->exps[k] > 0.0) || !std::isfinite(sh->exps[k]) || !std::isfinite(sh->coefs[k])) return ERI_E_INVALID;
    }
    return ERI_OK;
}

int64_t chunk_quartets_setting()
{
    int64_t q = int64_t(1) << 22;
    if (const char *cq = std::getenv("ERI_CHUNK_QUARTETS")) {
        const long long v = std::atoll(cq);
        if (v >= 1 && v <= (1LL << 26)) q = v;
    }
    return q;
}

// Plan build into an arena (after validation).  With a counting arena it only
// sizes; otherwise it returns the plan (host struct) whose device data live in
// the arena.
eri_plan *build_plan(const eri_shells *sh, int flags, const int32_t *quartets, int64_t nq, double tau, Arena &A,
                     hipStream_t s)
{
    std::unique_ptr<eri_plan> P(new eri_plan());
    P->flags = flags;
    P->sph = (flags & ERI_SPHERICAL) != 0;
    P->screened = quartets == nullptr;
    P->nshell = sh->nshell;
    BuildHost H;
    if (quartets) host_explicit(sh, flags, quartets, nq, H);
    else host_screened(sh, flags, chunk_quartets_setting(), H);
    BuildBufs X;
    plan_layout(A, P.get(), H, X);
    if (!A.base) return nullptr;
    const int ns = sh->nshell;
    HIP_CHECK(hipGetDevice(&P->device));
    {
        int ncu = 0;
        HIP_CHECK(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, P->device));
        P->grid_cap = std::max(1, ncu) * 8;
    }
    P->d_boys = boys_table(P->device);
    P->nbf = H.hbf[ns];
    P->hl.assign(sh->l, sh->l + ns);
    P->hk.assign(sh->nprim, sh->nprim + ns);
    P->hoff.assign(sh->prim_off, sh->prim_off + ns + 1);
    P->hcen.assign(sh->centers, sh->centers + 3 * (size_t)ns);
    P->hexp.assign(sh->exps, sh->exps + H.npr);
    P->hcn.resize(H.npr);
    upload(P->d_cen, sh->centers, (size_t)3 * ns, s);
    upload(P->d_l, sh->l, ns, s);
    upload(P->d_nprim, sh->nprim, ns, s);
    upload(P->d_off, sh->prim_off, ns + 1, s);
    upload(P->d_bf, H.hbf.data(), ns + 1, s);
    upload(P->d_nfun, H.hnf.data(), ns, s);
    upload(P->d_exps, sh->exps, H.npr, s);
    upload(X.raw, sh->coefs, H.npr, s);
    hipLaunchKernelGGL(k_normalize, dim3(nblk(ns, 128)), dim3(128), 0, s, ns, P->d_l, P->d_nprim, P->d_off, P->d_exps,
                       X.raw, P->d_cn, (flags & ERI_NO_NORMALIZE) ? 1 : 0);
    HIP_CHECK(hipGetLastError());
    HIP_CHECK(hipMemcpyAsync(P->hcn.data(), P->d_cn, sizeof(double) * H.npr, hipMemcpyDeviceToHost, s));
    if (quartets) build_explicit(P.get(), H, X, quartets, s);
    else build_screened(P.get(), H, X, tau, s);
    HIP_CHECK(hipStreamSynchronize(s));
    P->ws_used = A.used;
    return P.release();
}

// Index-map rows of plan slots [first, first + count) on the host.  A screened
// plan expands them on the device in pieces, into its chunk lists (calls on
// one plan do not overlap); synchronises the stream.
void fetch_rows(const eri_plan *P, int64_t first, int64_t count, std::vector<int> &rows, hipStream_t s)
{
    rows.resize(5 * (size_t)count);
    if (!P->screened) {
        if (count)
            HIP_CHECK(hipMemcpyAsync(rows.data(), P->d_qmap + 5 * first, sizeof(int) * 5 * count,
                                     hipMemcpyDeviceToHost, s));
        HIP_CHECK(hipStreamSynchronize(s));
        return;
    }
    const int64_t piece = std::max<int64_t>(1, (int64_t)ERI_LANES * 2 * P->chunk_q / 5);
    for (int64_t c = 0; c < count; c += piece) {
        const int64_t m = std::min(piece, count - c);
        hipLaunchKernelGGL(k_expand, dim3(nblk(m, 256)), dim3(256), 0, s, first + c, m, P->nent, P->d_ent_off, P->d_bd,
                           P->nbd, P->d_porder, P->d_pinfo, P->d_pair_i, (int *)nullptr, (int *)nullptr, P->d_chunk);
        HIP_CHECK(hipGetLastError());
        HIP_CHECK(hipMemcpyAsync(rows.data() + 5 * c, P->d_chunk, sizeof(int) * 5 * m, hipMemcpyDeviceToHost, s));
        HIP_CHECK(hipStreamSynchronize(s));
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

namespace {

// workspace argument check shared by the calls that take one: NULL asks for
// the size; otherwise *ws_bytes says how much is there and must cover `need`
int workspace_check(void *workspace, size_t *ws_bytes, size_t need)
{
    if (!workspace) {
        *ws_bytes = need;
        return 1;
    }
    if ((uintptr_t)workspace % 256 != 0) return ERI_E_INVALID;
    if (*ws_bytes < need) return ERI_E_WORKSPACE;
    return 0;
}

}  // namespace

extern "C" int eri_build_quartets(const eri_shells *sh, int flags, const int32_t *quartets, int64_t nq, double tau,
                                  void *workspace, size_t *ws_bytes, void *stream, eri_plan **plan)
{
    if (!ws_bytes || (workspace && !plan)) return ERI_E_INVALID;
    if (workspace) *plan = nullptr;
    int rc = validate_shells(sh);
    if (rc != ERI_OK) return rc;
    if (flags & ~(ERI_SPHERICAL | ERI_NO_NORMALIZE)) return ERI_E_INVALID;
    if (!(tau >= 0.0) || std::isinf(tau)) return ERI_E_INVALID;
    if (quartets && (nq < 0 || tau != 0.0)) return ERI_E_INVALID;
    if (quartets && nq > ((int64_t)1 << 30)) return ERI_E_UNSUPPORTED;
    const int ns = sh->nshell;
    if (quartets)
        for (int64_t x = 0; x < 4 * nq; ++x)
            if (quartets[x] < 0 || quartets[x] >= ns) return ERI_E_INVALID;
    if (!quartets && (int64_t)ns * (ns + 1) / 2 > (int64_t)INT32_MAX / 2) return ERI_E_UNSUPPORTED;
    try {
        Arena count;
        build_plan(sh, flags, quartets, nq, tau, count, (hipStream_t)stream);
        const int w = workspace_check(workspace, ws_bytes, count.used);
        if (w) return w > 0 ? ERI_OK : w;
        Arena A(workspace, *ws_bytes);
        *plan = build_plan(sh, flags, quartets, nq, tau, A, (hipStream_t)stream);
    } catch (const HipFail &f) {
        return translate(f);
    } catch (const WsShort &) {
        return ERI_E_WORKSPACE;
    } catch (const std::bad_alloc &) {
        return ERI_E_NOMEM;
    }
    return ERI_OK;
}

extern "C" int eri_plan_destroy(eri_plan *plan)
{
    delete plan;
    return ERI_OK;
}

extern "C" int eri_plan_set_streams(eri_plan *P, void *const *streams, int32_t n)
{
    if (!P || n < 0 || n > ERI_MAX_SIDE_STREAMS || (n > 0 && !streams)) return ERI_E_INVALID;
    for (int i = 0; i < n; ++i)
        if (!streams[i]) return ERI_E_INVALID;
    try {
        if (n > 0 && !P->ev_fork) {
            HIP_CHECK(hipEventCreateWithFlags(&P->ev_fork, hipEventDisableTiming));
            for (int i = 0; i < ERI_MAX_SIDE_STREAMS; ++i)
                HIP_CHECK(hipEventCreateWithFlags(&P->ev_side[i], hipEventDisableTiming));
        }
    } catch (const HipFail &f) {
        return translate(f);
    }
    P->nside = n;
    for (int i = 0; i < ERI_MAX_SIDE_STREAMS; ++i) P->side[i] = i < n ? (hipStream_t)streams[i] : nullptr;
    return ERI_OK;
}

extern "C" int eri_plan_info(const eri_plan *P, int64_t *nq, int64_t *nout, int32_t *nb, int32_t *nbf, int64_t *np)
{
    if (!P) return ERI_E_INVALID;
    if (nq) *nq = P->nq;
    if (nout) *nout = P->nout;
    if (nb) *nb = (int32_t)P->blocks.size();
    if (nbf) *nbf = P->nbf;
    if (np) *np = P->npairs;
    return ERI_OK;
}

extern "C" int eri_plan_blocks(const eri_plan *P, int32_t *cid, int64_t *start, int64_t *count, int64_t *out_off)
{
    if (!P) return ERI_E_INVALID;
    for (size_t b = 0; b < P->blocks.size(); ++b) {
        if (cid) cid[b] = P->blocks[b].cid;
        if (start) start[b] = P->blocks[b].start;
        if (count) count[b] = P->blocks[b].count;
        if (out_off) out_off[b] = P->blocks[b].out_off;
    }
    return ERI_OK;
}

extern "C" int eri_plan_quartets(const eri_plan *P, int64_t first, int64_t count, int32_t *dst, void *stream)
{
    if (!P || first < 0 || count < 0 || first > P->nq || count > P->nq - first) return ERI_E_INVALID;
    if (count == 0) return ERI_OK;
    if (!dst || count > (int64_t)INT32_MAX) return ERI_E_INVALID;
    hipStream_t s = (hipStream_t)stream;
    try {
        if (P->screened) {
            hipLaunchKernelGGL(k_expand, dim3(nblk(count, 256)), dim3(256), 0, s, first, count, P->nent, P->d_ent_off,
                               P->d_bd, P->nbd, P->d_porder, P->d_pinfo, P->d_pair_i, (int *)nullptr, (int *)nullptr,
                               dst);
            HIP_CHECK(hipGetLastError());
        } else {
            HIP_CHECK(hipMemcpyAsync(dst, P->d_qmap + 5 * first, sizeof(int) * 5 * count, hipMemcpyDeviceToDevice, s));
        }
    } catch (const HipFail &f) {
        return translate(f);
    }
    return ERI_OK;
}

extern "C" int eri_plan_index_map(const eri_plan *P, int32_t *dst, void *stream)
{
    if (!P || (!dst && P->nq)) return ERI_E_INVALID;
    if (!P->nq) return ERI_OK;
    if (P->nq > (int64_t)INT32_MAX) return ERI_E_UNSUPPORTED;
    return eri_plan_quartets(P, 0, P->nq, dst, stream);
}

extern "C" int eri_plan_schwarz(const eri_plan *P, double *dst, void *stream)
{
    if (!P || !dst) return ERI_E_INVALID;
    if (!P->screened) return ERI_E_UNSUPPORTED;
    hipError_t e = hipMemcpyAsync(dst, P->d_S, sizeof(double) * P->npairs, hipMemcpyDeviceToDevice, (hipStream_t)stream);
    if (e != hipSuccess) {
        g_last_error = std::string("hipMemcpyAsync: ") + hipGetErrorString(e);
        return ERI_E_HIP;
    }
    return ERI_OK;
}

extern "C" int eri_compute_batch(const eri_plan *P, int32_t b0, int32_t b1, double *out, int64_t cap, void *stream)
{
    if (!P) return ERI_E_INVALID;
    const int nb = (int)P->blocks.size();
    if (b0 < 0 || b1 > nb || b0 > b1) return ERI_E_INVALID;
    if (b0 == b1) return ERI_OK;
    const int64_t base = P->blocks[b0].out_off;
    const int64_t end = (b1 < nb) ? P->blocks[b1].out_off : P->nout;
    if (!out || cap < end - base) return out ? ERI_E_CAPACITY : ERI_E_INVALID;
    try {
        const hipStream_t s = (hipStream_t)stream;
        const int lanes = b1 - b0 > 1 ? lanes_of(P) : 1;
        if (lanes > 1) side_fork(P, s, lanes);
        int rr = 0;
        for (int b = b0; b < b1; ++b) {
            const EriBlock &B = P->blocks[b];
            const int lane = uses_scratch(P, B.cid) ? 0 : (rr++) % lanes;
            compute_range(P, B, 0, B.count, out + (B.out_off - base), lane_stream(P, lane, s), lane);
        }
        if (lanes > 1) side_join(P, s, lanes);
    } catch (const HipFail &f) {
        return translate(f);
    }
    return ERI_OK;
}

extern "C" int eri_compute_range(const eri_plan *P, int32_t block, int64_t first, int64_t count, double *out,
                                 int64_t cap, void *stream)
{
    if (!P || block < 0 || block >= (int)P->blocks.size() || first < 0 || count < 0) return ERI_E_INVALID;
    const EriBlock &B = P->blocks[block];
    if (first > B.count || count > B.count - first) return ERI_E_INVALID;
    if (count == 0) return ERI_OK;
    const int64_t need = count * (int64_t)B.na * B.nb * B.nc * B.nd;
    if (!out) return ERI_E_INVALID;
    if (cap < need) return ERI_E_CAPACITY;
    try {
        compute_range(P, B, first, count, out, (hipStream_t)stream, 0);
    } catch (const HipFail &f) {
        return translate(f);
    }
    return ERI_OK;
}

namespace {

int digest_entry(const eri_plan *P, const double *D, int32_t ldd, double *J, int32_t ldj, double *K, int32_t ldk,
                 bool wantJ, bool wantK, void *workspace, size_t *ws_bytes, void *stream,
                 DigestRange rg = DigestRange(), bool accumulate = false)
{
    if (!P || !ws_bytes) return ERI_E_INVALID;
    if (!P->screened) return ERI_E_UNSUPPORTED;
    if (wantK && P->nshell > 46340) return ERI_E_UNSUPPORTED;  // target block keys are nshell^2 in 32 bits
    try {
        const DigestShape d = digest_shape(P, wantJ, wantK);
        std::vector<ChunkLane> L;
        double *kacc = nullptr;
        Arena count;
        digest_layout(count, P, wantJ, wantK, d, L, &kacc);
        const int w = workspace_check(workspace, ws_bytes, count.used);
        if (w) return w > 0 ? ERI_OK : w;
        if (!D || ldd < P->nbf || (wantJ && (!J || ldj < P->nbf)) || (wantK && (!K || ldk < P->nbf)))
            return ERI_E_INVALID;
        Arena A(workspace, *ws_bytes);
        digest_JK_run(P, D, ldd, wantJ ? J : nullptr, ldj, wantK ? K : nullptr, ldk, A, (hipStream_t)stream, nullptr,
                      rg, accumulate);
    } catch (const HipFail &f) {
        return translate(f);
    } catch (const WsShort &) {
        return ERI_E_WORKSPACE;
    }
    return ERI_OK;
}

}  // namespace

extern "C" int eri_digest_J(const eri_plan *P, const double *D, int32_t ldd, double *J, int32_t ldj, void *workspace,
                            size_t *ws_bytes, void *stream)
{
    return digest_entry(P, D, ldd, J, ldj, nullptr, 0, true, false, workspace, ws_bytes, stream);
}

extern "C" int eri_digest_J_range(const eri_plan *P, int32_t block, int64_t first, int64_t count, const double *D,
                                  int32_t ldd, double *J, int32_t ldj, void *workspace, size_t *ws_bytes, void *stream)
{
    if (!P || block < 0 || block >= (int32_t)P->blocks.size() || first < 0 || count < 0) return ERI_E_INVALID;
    if (first > P->blocks[block].count || count > P->blocks[block].count - first) return ERI_E_INVALID;
    DigestRange rg;
    rg.block = block;
    rg.first = first;
    rg.count = count;
    return digest_entry(P, D, ldd, J, ldj, nullptr, 0, true, false, workspace, ws_bytes, stream, rg, true);
}

extern "C" int eri_digest_JK(const eri_plan *P, const double *D, int32_t ldd, double *J, int32_t ldj, double *K,
                             int32_t ldk, void *workspace, size_t *ws_bytes, void *stream)
{
    if (!J && !K) return ERI_E_INVALID;
    return digest_entry(P, D, ldd, J, ldj, K, ldk, J != nullptr, K != nullptr, workspace, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// J digestion that allocates nothing, for callers that cannot allocate
// ---------------------------------------------------------------------------
// Its chunk buffers live in `scratch`, a file-scope device array of
// ERI_NOALLOC_SCRATCH_BYTES that every device holds until the process ends.
// Host code never passes the array's name to a kernel (on the host it is only
// a stand-in): the device address of each device's copy is looked up once, with
// that device current, and kept in g_scratch_dev.
static __device__ __align__(256) unsigned char scratch[ERI_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
std::vector<void *> g_scratch_dev;

int scratch_on_current_device(void **ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        g_last_error = std::string("hipGetDevice: ") + hipGetErrorString(e);
        return ERI_E_HIP;
    }
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if ((int)g_scratch_dev.size() <= dev) g_scratch_dev.resize(dev + 1, nullptr);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            g_last_error = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
            return ERI_E_HIP;
        }
        g_scratch_dev[dev] = p;
    }
    *ptr = g_scratch_dev[dev];
    return ERI_OK;
}

}  // namespace

extern "C" int eri_digest_J_noalloc(const eri_plan *P, const double *D, int32_t ldd, double *J, int32_t ldj,
                                    void *stream)
{
    if (!P || !D || !J || ldd < P->nbf || ldj < P->nbf) return ERI_E_INVALID;
    if (!P->screened) return ERI_E_UNSUPPORTED;
    try {
        int dev = 0;
        HIP_CHECK(hipGetDevice(&dev));
        if (dev != P->device) return ERI_E_INVALID;
        DigestShape d;
        if (!digest_shape_capped(P, true, false, ERI_NOALLOC_SCRATCH_BYTES, d)) {
            g_last_error = "the plan's largest class block needs more than ERI_NOALLOC_SCRATCH_BYTES";
            return ERI_E_WORKSPACE;
        }
        void *ptr = nullptr;
        const int rc = scratch_on_current_device(&ptr);
        if (rc != ERI_OK) return rc;
        Arena A(ptr, ERI_NOALLOC_SCRATCH_BYTES);
        digest_JK_run(P, D, ldd, J, ldj, nullptr, 0, A, (hipStream_t)stream, &d);
    } catch (const HipFail &f) {
        return translate(f);
    } catch (const WsShort &) {
        return ERI_E_WORKSPACE;
    }
    return ERI_OK;
}

// ---------------------------------------------------------------------------
// First derivatives with respect to the centres
// ---------------------------------------------------------------------------
namespace {

// Everything a derivative call needs, from the slots' index-map rows.
struct DerivHost {
    std::vector<int> rows;                 // [5 count]
    std::vector<int64_t> dst_off, cart_off;
    int64_t dtot = 0, ctot = 0;
    // auxiliary shells: [0, ns) the shells, [ns, 2ns) raised, [2ns, 3ns) lowered (raw coefficients)
    std::vector<int32_t> al, ak, aoff, aq, umap;
    std::vector<double> acen, aexp, acf;
    eri_shells ash{};
    int64_t aux_nout = 0;
    // the auxiliary plan's quartet count, primitive pair total and classes
    int64_t na = 0, nppd = 0;
    bool present[ERI_NCLASS] = {};
};

// list: fill the auxiliary quartet list (aq, umap); a size query needs only its counts
int deriv_host(const eri_plan *P, int64_t first, int64_t count, hipStream_t s, DerivHost &H, bool list)
{
    fetch_rows(P, first, count, H.rows, s);
    const int ns = P->nshell;
    const std::vector<int> &hl = P->hl, &hk = P->hk, &hoff = P->hoff;
    // every auxiliary class (one shell raised or lowered) must be in the library;
    // the flags set here are the auxiliary plan's classes
    bool *checked = H.present;
    int prev[4] = {-1, -1, -1, -1};
    for (int64_t t = 0; t < count; ++t) {
        const int *r = &H.rows[5 * t];
        const int lt[4] = {hl[r[0]], hl[r[1]], hl[r[2]], hl[r[3]]};
        if (lt[0] == prev[0] && lt[1] == prev[1] && lt[2] == prev[2] && lt[3] == prev[3]) continue;
        for (int k = 0; k < 4; ++k) prev[k] = lt[k];
        for (int p = 0; p < 4; ++p)
            for (int dl = -1; dl <= 1; dl += 2) {
                if (dl < 0 && lt[p] == 0) continue;  // no lowered quartet for an s shell
                int l4[4] = {lt[0], lt[1], lt[2], lt[3]};
                l4[p] += dl;
                const int cid = class_of(l4[0], l4[1], l4[2], l4[3]);
                if (checked[cid]) continue;
                if (!find_class(cid, false)) return ERI_E_UNSUPPORTED;
                checked[cid] = true;
            }
    }
    const bool sph = P->sph;
    H.dst_off.resize(count);
    H.cart_off.resize(count);
    for (int64_t t = 0; t < count; ++t) {
        const int *r = &H.rows[5 * t];
        int64_t nf = 1, nc = 1;
        for (int k = 0; k < 4; ++k) {
            nf *= nfun(hl[r[k]], sph);
            nc *= ncart(hl[r[k]]);
        }
        H.dst_off[t] = H.dtot;
        H.cart_off[t] = H.ctot;
        H.dtot += 12 * nf;
        H.ctot += 12 * nc;
    }
    const int npr = hoff[ns];
    H.al.resize(3 * ns);
    H.ak.resize(3 * ns);
    H.aoff.resize(3 * ns + 1);
    H.acen.resize(9 * (size_t)ns);
    H.aexp.resize(3 * (size_t)npr);
    H.acf.resize(3 * (size_t)npr);
    H.aoff[0] = 0;
    for (int part = 0; part < 3; ++part)
        for (int x = 0; x < ns; ++x) {
            const int y = part * ns + x;
            H.al[y] = part == 0 ? hl[x] : part == 1 ? hl[x] + 1 : std::max(hl[x] - 1, 0);
            H.ak[y] = hk[x];
            H.aoff[y + 1] = H.aoff[y] + hk[x];
            for (int c = 0; c < 3; ++c) H.acen[3 * y + c] = P->hcen[3 * x + c];
            for (int q = 0; q < hk[x]; ++q) {
                const double a = P->hexp[hoff[x] + q], c = P->hcn[hoff[x] + q];
                H.aexp[H.aoff[y] + q] = a;
                H.acf[H.aoff[y] + q] = part == 0 ? c : part == 1 ? 2.0 * a * c : (hl[x] > 0 ? c : 0.0);
            }
        }
    H.ash = eri_shells{3 * ns, H.acen.data(), H.al.data(), H.ak.data(), H.aoff.data(), H.aexp.data(), H.acf.data()};
    // slot t, centre p, raised (0) or lowered (1): derivative index u = (t 4 + p) 2 + sg.
    // An s shell has no lowered term (every exponent of the centre is zero), so
    // its lowered quartet is not listed; umap holds the u of every listed quartet.
    std::vector<int64_t> anc(3 * (size_t)ns);
    for (int y = 0; y < 3 * ns; ++y) anc[y] = ncart(H.al[y]);
    int64_t na = 0;
    for (int64_t t = 0; t < count; ++t) {
        const int *r = &H.rows[5 * t];
        int n = 0;
        for (int p = 0; p < 4; ++p) n += hl[r[p]] > 0 ? 2 : 1;
        na += n;
        // raised and lowered shells keep their primitive counts
        H.nppd += n * ((int64_t)hk[r[0]] * hk[r[1]] + (int64_t)hk[r[2]] * hk[r[3]]);
    }
    H.na = na;
    if (!list) {
        for (int64_t t = 0; t < count; ++t) {
            const int *r = &H.rows[5 * t];
            for (int p = 0; p < 4; ++p)
                for (int sg = 0; sg < 2; ++sg) {
                    if (sg == 1 && hl[r[p]] == 0) continue;
                    int64_t blk = 1;
                    for (int k = 0; k < 4; ++k) blk *= anc[r[k] + (k == p ? (sg == 0 ? 1 : 2) * ns : 0)];
                    H.aux_nout += blk;
                }
        }
        return ERI_OK;
    }
    H.aq.resize(4 * (size_t)na);
    H.umap.resize((size_t)na);
    int64_t x = 0;
    for (int64_t t = 0; t < count; ++t) {
        const int *r = &H.rows[5 * t];
        for (int p = 0; p < 4; ++p)
            for (int sg = 0; sg < 2; ++sg) {
                if (sg == 1 && hl[r[p]] == 0) continue;
                int32_t *q = &H.aq[4 * (size_t)x];
                for (int k = 0; k < 4; ++k) q[k] = r[k];
                q[p] += (sg == 0 ? 1 : 2) * ns;
                H.aux_nout += anc[q[0]] * anc[q[1]] * anc[q[2]] * anc[q[3]];
                H.umap[x++] = (int32_t)((t * 4 + p) * 2 + sg);
            }
    }
    return ERI_OK;
}

struct DerivBufs {
    int *rows = nullptr, *umap = nullptr;
    double *aux = nullptr, *cart = nullptr, *tmp = nullptr;
    int64_t *slot_of = nullptr, *bt = nullptr, *aux_off = nullptr, *off = nullptr;
};

void deriv_layout(Arena &A, const eri_plan *P, int64_t count, const DerivHost &H, DerivBufs &X)
{
    X.rows = A.take<int>(5 * (size_t)count);
    X.umap = A.take<int>(H.na);
    X.aux = A.take<double>(H.aux_nout);
    X.slot_of = A.take<int64_t>(8 * (size_t)count);
    X.bt = A.take<int64_t>(3 * ERI_NCLASS);
    X.aux_off = A.take<int64_t>(H.na);
    X.off = A.take<int64_t>(2 * (size_t)count);
    if (P->sph) {
        X.cart = A.take<double>(H.ctot);
        X.tmp = A.take<double>(H.ctot);
    }
}

}  // namespace

extern "C" int eri_compute_deriv(const eri_plan *P, int64_t first, int64_t count, double *out, int64_t cap,
                                 void *workspace, size_t *ws_bytes, void *stream)
{
    if (!P || !ws_bytes || first < 0 || count < 0 || first > P->nq || count > P->nq - first) return ERI_E_INVALID;
    if (count > ((int64_t)1 << 24)) return ERI_E_INVALID;
    if (count == 0) {
        if (!workspace) *ws_bytes = 0;
        return ERI_OK;
    }
    hipStream_t s = (hipStream_t)stream;
    std::unique_ptr<eri_plan> Aux;
    try {
        DerivHost H;
        int rc = deriv_host(P, first, count, s, H, workspace != nullptr);
        if (rc != ERI_OK) return rc;
        DerivBufs X;
        Arena cnt;
        const int64_t na = H.na;
        {
            BuildHost BH;
            host_explicit_counts(&H.ash, ERI_NO_NORMALIZE, na, H.nppd, H.present, BH);
            eri_plan L;
            L.flags = ERI_NO_NORMALIZE;
            L.nshell = H.ash.nshell;
            BuildBufs LX;
            plan_layout(cnt, &L, BH, LX);
        }
        deriv_layout(cnt, P, count, H, X);
        const int w = workspace_check(workspace, ws_bytes, cnt.used);
        if (w) return w > 0 ? ERI_OK : w;
        if (!out) return ERI_E_INVALID;
        if (cap < H.dtot) return ERI_E_CAPACITY;
        Arena A(workspace, *ws_bytes);
        Aux.reset(build_plan(&H.ash, ERI_NO_NORMALIZE, H.aq.data(), na, 0.0, A, s));
        deriv_layout(A, P, count, H, X);
        const eri_plan *Ap = Aux.get();
        for (const EriBlock &B : Ap->blocks) compute_range(Ap, B, 0, B.count, X.aux + B.out_off, s, 0);
        upload(X.rows, H.rows.data(), 5 * (size_t)count, s);
        upload(X.umap, H.umap.data(), (size_t)na, s);
        hipLaunchKernelGGL(k_invert_src, dim3(nblk(na, 256)), dim3(256), 0, s, na, Ap->d_qsrc, X.umap, X.slot_of);
        HIP_CHECK(hipGetLastError());
        const int nb = (int)Ap->blocks.size();
        std::vector<int64_t> bt(3 * (size_t)nb);
        for (int b = 0; b < nb; ++b) {
            const EriBlock &B = Ap->blocks[b];
            bt[b] = B.start;
            bt[nb + b] = B.out_off;
            bt[2 * nb + b] = (int64_t)B.na * B.nb * B.nc * B.nd;
        }
        upload(X.bt, bt.data(), bt.size(), s);
        hipLaunchKernelGGL(k_slot_offsets, dim3(nblk(na, 256)), dim3(256), 0, s, na, nb, X.bt, X.bt + nb, X.bt + 2 * nb,
                           X.aux_off);
        HIP_CHECK(hipGetLastError());
        upload(X.off, H.dst_off.data(), count, s);
        upload(X.off + count, H.cart_off.data(), count, s);
        // threads per item: the smallest power of two (at most 256) covering the
        // largest Cartesian block of the call, so that small classes share a workgroup
        int64_t max_ncar = 1;
        for (int64_t t = 0; t < count; ++t) {
            int64_t nc = 1;
            for (int k = 0; k < 4; ++k) nc *= ncart(P->hl[H.rows[5 * t + k]]);
            max_ncar = std::max(max_ncar, nc);
        }
        auto tpi_for = [](int64_t work) {
            int v = 1;
            while (v < 256 && v < work) v *= 2;
            return v;
        };
        const int tpc = tpi_for(12 * max_ncar), tps = tpi_for(max_ncar);
        const int64_t nwc = (count + 256 / tpc - 1) / (256 / tpc), nws = (12 * count + 256 / tps - 1) / (256 / tps);
        if (!P->sph) {
            hipLaunchKernelGGL(k_deriv_combine, dim3((unsigned)nwc), dim3(256), 0, s, count, tpc, X.rows, P->d_l,
                               X.slot_of, Ap->d_qmap, Ap->d_l, X.aux_off, X.aux, X.off, out);
        } else {
            hipLaunchKernelGGL(k_deriv_combine, dim3((unsigned)nwc), dim3(256), 0, s, count, tpc, X.rows, P->d_l,
                               X.slot_of, Ap->d_qmap, Ap->d_l, X.aux_off, X.aux, X.off + count, X.cart);
            HIP_CHECK(hipGetLastError());
            // blocks staged in LDS where two buffers per item fit 64 KB per workgroup
            const size_t lds = (size_t)(256 / tps) * 2 * max_ncar * sizeof(double);
            if (lds <= 65536)
                hipLaunchKernelGGL(k_deriv_sph_lds, dim3((unsigned)nws), dim3(256), lds, s, count, tps, (int)max_ncar,
                                   X.rows, P->d_l, X.cart, X.off + count, X.off, out);
            else
                hipLaunchKernelGGL(k_deriv_sph, dim3((unsigned)nws), dim3(256), 0, s, count, tps, X.rows, P->d_l,
                                   X.cart, X.tmp, X.off + count, X.off, out);
        }
        HIP_CHECK(hipGetLastError());
        // the host vectors uploaded above are read by the copies before they return
        HIP_CHECK(hipStreamSynchronize(s));
    } catch (const HipFail &f) {
        return translate(f);
    } catch (const WsShort &) {
        return ERI_E_WORKSPACE;
    } catch (const std::bad_alloc &) {
        return ERI_E_NOMEM;
    }
    return ERI_OK;
}

extern "C" const char *eri_strerror(int code)
{
    switch (code) {
    case ERI_OK: return "ok";
    case ERI_E_INVALID: return "invalid argument";
    case ERI_E_UNSUPPORTED: return "unsupported";
    case ERI_E_CAPACITY: return "output buffer too small";
    case ERI_E_HIP: {
        static thread_local std::string msg;
        msg = "HIP error: " + g_last_error;
        return msg.c_str();
    }
    case ERI_E_NOMEM: return "out of host memory";
    case ERI_E_WORKSPACE: return "workspace smaller than the size query returned";
    default: return "unknown error";
    }
}

extern "C" int eri_fp64_fma_tflops(double *tflops, void *stream)
{
    if (!tflops) return ERI_E_INVALID;
    hipStream_t s = (hipStream_t)stream;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    int rc = ERI_OK;
    try {
        int dev = 0, ncu = 0;
        HIP_CHECK(hipGetDevice(&dev));
        HIP_CHECK(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev));
        const int grid = ncu * 8;  // 256-lane workgroups: 8 per compute unit = 8 waves per SIMD
        double *sink = nullptr;
        HIP_CHECK(hipGetSymbolAddress((void **)&sink, HIP_SYMBOL(g_fma_sink)));
        HIP_CHECK(hipEventCreate(&e0));
        HIP_CHECK(hipEventCreate(&e1));
        hipLaunchKernelGGL(k_fma_rate, dim3(grid), dim3(256), 0, s, sink, 0.999, 1e-3, -1.0);
        HIP_CHECK(hipGetLastError());
        const int reps = 5;
        HIP_CHECK(hipEventRecord(e0, s));
        for (int r = 0; r < reps; ++r) hipLaunchKernelGGL(k_fma_rate, dim3(grid), dim3(256), 0, s, sink, 0.999, 1e-3, -1.0);
        HIP_CHECK(hipGetLastError());
        HIP_CHECK(hipEventRecord(e1, s));
        HIP_CHECK(hipEventSynchronize(e1));
        float ms = 0.f;
        HIP_CHECK(hipEventElapsedTime(&ms, e0, e1));
        const double flop = 2.0 * FMA_CHAINS * FMA_ITERS * (double)grid * 256 * reps;
        *tflops = flop / (ms * 1e-3) / 1e12;
    } catch (const HipFail &f) {
        rc = translate(f);
    }
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    return rc;
}

extern "C" int eri_class_info(int32_t cid, int32_t *l4, int32_t *tier)
{
    const EriClassEntry *ce = find_class(cid, true);
    if (!ce) return ERI_E_INVALID;
    if (l4) {
        l4[0] = ce->la;
        l4[1] = ce->lb;
        l4[2] = ce->lc;
        l4[3] = ce->ld;
    }
    if (tier) *tier = ce->tier;
    return ERI_OK;
}
