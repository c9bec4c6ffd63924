/*
 * eri_oracle.c -- plain, slow, fp64 CPU reference for four-centre electron
 * repulsion integrals over contracted Cartesian Gaussian shells.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark load it.  It shares no code, tables or constants with
 * the HIP path.
 *
 * Source: "FusionRCG: Orchestrating Recursive Computation Graphs across GPU
 * Memory Hierarchies" (Wei, Zhang, Chen, Ju, Hu, Yang, Xia).  What is computed:
 *   - the integral (ab|cd) of its Eq. (1), section II-A, over Cartesian
 *     Gaussians phi_a = x^ax y^ay z^az exp(-alpha r_A^2);
 *   - the contraction over primitive quartets of Algorithm 2 (section III-C);
 *   - the Cartesian-to-spherical shell transform of Eq. (8) (section III-B)
 *     applied to all four indices of the finished Cartesian block, i.e. the
 *     materialise-then-transform form of Eq. (17);
 *   - the Coulomb matrix J = sum (mu nu|la si) D_la_si that Algorithm 2 scatters.
 * The page does not print how F_m(T) is evaluated, how primitives are
 * normalised, the spherical coefficients, or any screening rule; the readings
 * taken here are stated next to each function.
 *
 * Method (deliberately NOT the HGP split the GPU path uses): the four-index
 * Obara-Saika recurrence, which may raise any of a, b, c, d, filled bottom-up
 * in a dense table for every primitive quartet.  No horizontal recurrence is
 * used.  Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC.
 *
 * Precision: all arithmetic is done in the type `real`, fp64 by default.
 * Built with -DORACLE_QUAD the same source computes in IEEE binary128
 * (__float128, libquadmath) and rounds only the results to fp64.  That build
 * exists to adjudicate: it shows how far the fp64 oracle itself is from the
 * exact value of the same definition.  Inputs and outputs stay fp64 in both.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#ifdef ORACLE_QUAD
#include <quadmath.h>
typedef __float128 real;
#define R_EXP expq
#define R_SQRT sqrtq
#define R_POW powq
#define R_ERF erfq
#define R_FABS fabsq
#define R_PI M_PIq
#define R_SERIES_TOL 1e-36Q
#else
typedef double real;
#define R_EXP exp
#define R_SQRT sqrt
#define R_POW pow
#define R_ERF erf
#define R_FABS fabs
#define R_PI M_PI
#define R_SERIES_TOL 1e-18
#endif

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0 /* >0 only in test builds that plant a known mistake */
#endif
#define OR_LMAX 10 /* largest shell l the oracle accepts (4, plus headroom for the finite-difference
                      pins and the intermediates (e_A s_B| of the two-phase floor, |e| <= 9) */
#define OR_MMAX (4 * (OR_LMAX + 1))
#define OR_NCART ((OR_LMAX + 2) * (OR_LMAX + 3) / 2)                  /* components of l <= OR_LMAX + 1 */
#define OR_NTRIP ((OR_LMAX + 2) * (OR_LMAX + 3) * (OR_LMAX + 4) / 6)  /* triples of total <= OR_LMAX + 1 */

enum { OR_SPHERICAL = 1, OR_NO_NORMALIZE = 2 };

/* ------------------------------------------------------------------------ */
/* Boys function F_m(T) = int_0^1 t^(2m) exp(-T t^2) dt                       */
/* ------------------------------------------------------------------------ */
/* Reading (the page calls F_m(T) the seed of the recurrence, Eq. (2)
 * preamble, but gives no evaluation method):
 *   T <= OR_BOYS_SWITCH: the series
 *        F_M(T) = exp(-T) * sum_k (2T)^k / ((2M+1)(2M+3)...(2M+2k+1))
 *     for the highest order M, then downward recursion
 *        F_m = (2T F_{m+1} + exp(-T)) / (2m+1).
 *   T >  OR_BOYS_SWITCH: F_0 = sqrt(pi/T) erf(sqrt T) / 2 and upward recursion
 *        F_{m+1} = ((2m+1) F_m - exp(-T)) / (2T),
 *     which is well conditioned there because (2m+1)F_m >> exp(-T).        */
#define OR_BOYS_SWITCH 50.0

static void boys_r(int mmax, real T, real *F)
{
    if (T <= OR_BOYS_SWITCH) {
        real e = R_EXP(-T);
        real term = 1.0 / (2.0 * mmax + 1.0);
        real sum = term;
        for (int k = 1; k < 100000; ++k) {
            term *= 2.0 * T / (2.0 * mmax + 2.0 * k + 1.0);
            sum += term;
            if (term < R_SERIES_TOL * sum && k > T) break;
        }
        F[mmax] = e * sum;
        for (int m = mmax - 1; m >= 0; --m)
            F[m] = (2.0 * T * F[m + 1] + e) / (2.0 * m + 1.0 + (ORACLE_MUTANT == 4 ? 2.0 : 0.0));
    } else {
        real e = R_EXP(-T);
        F[0] = 0.5 * R_SQRT(R_PI / T) * R_ERF(R_SQRT(T));
        for (int m = 0; m < mmax; ++m)
            F[m + 1] = ((2.0 * m + 1.0) * F[m] - e) / (2.0 * T);
    }
}

void oracle_boys(int mmax, double T, double *F)
{
    real Fr[OR_MMAX + 1];
    if (mmax < 0 || mmax > OR_MMAX) return;
    boys_r(mmax, T, Fr);
    for (int m = 0; m <= mmax; ++m) F[m] = (double)Fr[m];
}

/* ------------------------------------------------------------------------ */
/* Cartesian components                                                      */
/* ------------------------------------------------------------------------ */
/* Order within a shell of angular momentum l: x-power descending, then
 * y-power descending (d: xx, xy, xz, yy, yz, zz).                           */
static int ncart(int l) { return (l + 1) * (l + 2) / 2; }
static int nsph(int l) { return 2 * l + 1; }

static void cart_list(int l, int (*c)[3])
{
    int n = 0;
    for (int i = l; i >= 0; --i)
        for (int j = l - i; j >= 0; --j) {
            c[n][0] = i;
            c[n][1] = j;
            c[n][2] = l - i - j;
            ++n;
        }
}

/* All exponent triples with total <= L, ordered by total then the order above. */
typedef struct {
    int n;
    int t[OR_NTRIP][3];
    int idx[OR_LMAX + 2][OR_LMAX + 2][OR_LMAX + 2];
} tripset;

static void tripset_init(tripset *s, int L)
{
    s->n = 0;
    for (int i = 0; i < OR_LMAX + 2; ++i)
        for (int j = 0; j < OR_LMAX + 2; ++j)
            for (int k = 0; k < OR_LMAX + 2; ++k) s->idx[i][j][k] = -1;
    for (int tot = 0; tot <= L; ++tot) {
        int c[OR_NCART][3];
        cart_list(tot, c);
        for (int q = 0; q < ncart(tot); ++q) {
            s->t[s->n][0] = c[q][0];
            s->t[s->n][1] = c[q][1];
            s->t[s->n][2] = c[q][2];
            s->idx[c[q][0]][c[q][1]][c[q][2]] = s->n;
            s->n++;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Normalisation                                                             */
/* ------------------------------------------------------------------------ */
/* Reading (not on the page): each primitive gets
 *   N(alpha, l) = (2 alpha/pi)^(3/4) (4 alpha)^(l/2) / sqrt((2l-1)!!),
 * the same factor for every Cartesian component of the shell (it normalises
 * the x^l component); then the contracted x^l component is scaled to unit
 * norm using  int x^(2l) exp(-p r^2) = (pi/p)^(3/2) (2l-1)!! / (2p)^l.       */
static real dfact(int n) /* n!!, with (-1)!! = 1 */
{
    real r = 1.0;
    for (int k = n; k > 1; k -= 2) r *= k;
    return r;
}

static void normalize_r(int l, int K, const double *alpha, const double *c_in, real *c_out)
{
    for (int k = 0; k < K; ++k)
        c_out[k] = c_in[k] * R_POW(2.0 * (real)alpha[k] / R_PI, (real)0.75) *
                   R_POW(4.0 * (real)alpha[k], (real)(0.5 * l + (ORACLE_MUTANT == 6 ? 0.5 : 0.0))) /
                   R_SQRT(dfact(2 * l - 1));
    real s = 0.0;
    for (int k = 0; k < K; ++k)
        for (int q = 0; q < K; ++q) {
            real p = (real)alpha[k] + (real)alpha[q];
            s += c_out[k] * c_out[q] * R_POW(R_PI / p, (real)1.5) * dfact(2 * l - 1) / R_POW(2.0 * p, (real)l);
        }
    real f = 1.0 / R_SQRT(s);
    for (int k = 0; k < K; ++k) c_out[k] *= f;
}

void oracle_normalize(int l, int K, const double *alpha, const double *c_in, double *c_out)
{
    real *c = (real *)malloc(sizeof(real) * (K > 0 ? K : 1));
    normalize_r(l, K, alpha, c_in, c);
    for (int k = 0; k < K; ++k) c_out[k] = (double)c[k];
    free(c);
}

/* ------------------------------------------------------------------------ */
/* Spherical transform coefficients (Eq. (8); coefficients not printed)       */
/* ------------------------------------------------------------------------ */
/* Reading: real solid harmonics without Condon-Shortley phase, ordered
 * m = -l..l.  Unnormalised polynomial (closed form, sums over t, u, v):
 *   S_lm = sum_t sum_u sum_v C x^(2t+|m|-2(u+v)) y^(2(u+v)) z^(l-2t-|m|),
 *   C = (-1)^(t+v-vm) 4^(-t) binom(l,t) binom(l-t,|m|+t) binom(t,u) binom(|m|,2v),
 * with vm = 0 for m >= 0 (v integer) and vm = 1/2 for m < 0 (v half-integer).
 * Each row is then scaled so that T S_cart T^T = I for a shell normalised as
 * above; the leading monomial x^|m| z^(l-|m|) (m>0), x^(|m|-1) y z^(l-|m|)
 * (m<0) or z^l (m=0) comes out with a positive coefficient.                 */
static real binom(int n, int k)
{
    if (k < 0 || k > n) return 0.0;
    real r = 1.0;
    for (int i = 1; i <= k; ++i) r = r * (n - k + i) / i;
    return r;
}

/* one-centre overlap of two Cartesian components of the normalised shell */
static real cart_overlap(const int *p, const int *q, int l)
{
    int sx = p[0] + q[0], sy = p[1] + q[1], sz = p[2] + q[2];
    if ((sx | sy | sz) & 1) return 0.0;
    return dfact(sx - 1) * dfact(sy - 1) * dfact(sz - 1) / dfact(2 * l - 1);
}

/* T[(2l+1) x ncart(l)], row-major */
static void sph_coeffs_r(int l, real *T)
{
    int nc = ncart(l);
    int c[OR_NCART][3];
    cart_list(l, c);
    for (int mi = 0; mi < nsph(l); ++mi) {
        int m = mi - l, am = abs(m);
        real *row = T + (size_t)mi * nc;
        for (int q = 0; q < nc; ++q) row[q] = 0.0;
        /* 2v runs over even values (m >= 0) or odd values (m < 0) in [0, |m|] */
        for (int t = 0; t <= (l - am) / 2; ++t)
            for (int u = 0; u <= t; ++u)
                for (int twov = (m >= 0 ? 0 : 1); twov <= am; twov += 2) {
                    int sgn_exp = t + (ORACLE_MUTANT == 5 ? 0 : (twov - (m >= 0 ? 0 : 1)) / 2);
                    real coef = ((sgn_exp & 1) ? -1.0 : 1.0) * R_POW((real)0.25, (real)t) * binom(l, t) *
                                  binom(l - t, am + t) * binom(t, u) * binom(am, twov);
                    int px = 2 * t + am - 2 * u - twov;
                    int py = 2 * u + twov;
                    int pz = l - 2 * t - am;
                    if (px < 0 || pz < 0) continue;
                    for (int q = 0; q < nc; ++q)
                        if (c[q][0] == px && c[q][1] == py && c[q][2] == pz) row[q] += coef;
                }
        real nrm = 0.0;
        for (int p = 0; p < nc; ++p)
            for (int q = 0; q < nc; ++q) nrm += row[p] * row[q] * cart_overlap(c[p], c[q], l);
        real f = 1.0 / R_SQRT(nrm);
        for (int q = 0; q < nc; ++q) row[q] *= f;
    }
}

void oracle_sph_coeffs(int l, double *T)
{
    real Tr[(2 * OR_LMAX + 1) * OR_NCART];
    if (l < 0 || l > OR_LMAX) return;
    sph_coeffs_r(l, Tr);
    for (int q = 0; q < nsph(l) * ncart(l); ++q) T[q] = (double)Tr[q];
}

/* ------------------------------------------------------------------------ */
/* Four-index Obara-Saika for one contracted shell quartet (Cartesian)       */
/* ------------------------------------------------------------------------ */
/* The integral of Eq. (1).  Gaussian-product quantities (the page's zeta,
 * eta, rho, P, W of Eq. (2)):
 *   zeta = alpha+beta, eta = gamma+delta, rho = zeta eta/(zeta+eta),
 *   P = (alpha A + beta B)/zeta, Q = (gamma C + delta D)/eta,
 *   W = (zeta P + eta Q)/(zeta+eta), T = rho |P-Q|^2.
 * Base value (reading of "F_m(T) = [00|00]^(m)", which omits the prefactor):
 *   [00|00]^(m) = 2 pi^(5/2) / (zeta eta sqrt(zeta+eta))
 *                 exp(-alpha beta |AB|^2/zeta) exp(-gamma delta |CD|^2/eta) F_m(T).
 * Raising a by 1_i (b, c, d analogous; Obara & Saika 1986):
 *   [a+1i b|cd]^(m) = (P-A)_i [ab|cd]^(m) + (W-P)_i [ab|cd]^(m+1)
 *     + a_i/(2 zeta) ([a-1i b|cd]^(m) - rho/zeta [a-1i b|cd]^(m+1))
 *     + b_i/(2 zeta) ([a b-1i|cd]^(m) - rho/zeta [a b-1i|cd]^(m+1))
 *     + c_i/(2(zeta+eta)) [ab|c-1i d]^(m+1) + d_i/(2(zeta+eta)) [ab|c d-1i]^(m+1).
 * For a ket index the roles swap: (Q-C)_i, (W-Q)_i, 1/(2 eta), rho/eta, and
 * the cross terms carry a_i, b_i.  A table entry is reduced on the first of
 * a, b, c, d that is non-zero, along its first non-zero axis.              */
typedef struct {
    tripset ta, tb, tc, td;
    real *V;
    size_t cap;
} os_work;

static inline size_t vidx(const os_work *w, int ia, int ib, int ic, int id, int m, int M1)
{
    return ((((size_t)ia * w->tb.n + ib) * w->tc.n + ic) * w->td.n + id) * M1 + m;
}

/* dout == NULL: the integrals of the block into out.  dout != NULL: instead
 * the first derivatives with respect to the 12 centre coordinates (A_x A_y
 * A_z B_x ... D_z), block after block into dout.  Differentiating a primitive
 * Cartesian Gaussian with respect to its own centre gives
 *   d/dA_i [x_A^a_x y_A^a_y z_A^a_z exp(-alpha r_A^2)]
 *     = 2 alpha (component a+1_i) - a_i (component a-1_i),
 * so the table is filled one unit higher on every index and each derivative
 * element is that combination of primitive integrals, contracted like the
 * integrals themselves (the normalisation belongs to the undifferentiated
 * shell). */
static void os_quartet(os_work *w, const int l4[4], const double *cen[4], int K4[4],
                       const double *al[4], const real *cc[4], real *out, real *dout)
{
    int la = l4[0], lb = l4[1], lc = l4[2], ld = l4[3];
    const int ext = dout ? 1 : 0;
    int Lt = la + lb + lc + ld + 4 * ext, M1 = Lt + 1;
    tripset_init(&w->ta, la + ext);
    tripset_init(&w->tb, lb + ext);
    tripset_init(&w->tc, lc + ext);
    tripset_init(&w->td, ld + ext);
    size_t need = (size_t)w->ta.n * w->tb.n * w->tc.n * w->td.n * M1;
    if (need > w->cap) {
        free(w->V);
        w->V = (real *)malloc(need * sizeof(real));
        w->cap = need;
    }
    real *V = w->V;
    int ca[OR_NCART][3], cb[OR_NCART][3], ccc[OR_NCART][3], cd[OR_NCART][3];
    cart_list(la, ca);
    cart_list(lb, cb);
    cart_list(lc, ccc);
    cart_list(ld, cd);
    int na = ncart(la), nb = ncart(lb), nc = ncart(lc), nd = ncart(ld);
    size_t nout = (size_t)na * nb * nc * nd;
    if (dout)
        for (size_t q = 0; q < 12 * nout; ++q) dout[q] = 0.0;
    else
        for (size_t q = 0; q < nout; ++q) out[q] = 0.0;
    const double *A = cen[0], *B = cen[1], *C = cen[2], *D = cen[3];
    real AB2 = 0, CD2 = 0;
    for (int i = 0; i < 3; ++i) {
        AB2 += ((real)A[i] - B[i]) * ((real)A[i] - B[i]);
        CD2 += ((real)C[i] - D[i]) * ((real)C[i] - D[i]);
    }
    real F[OR_MMAX + 1];

    for (int pa = 0; pa < K4[0]; ++pa)
        for (int pb = 0; pb < K4[1]; ++pb)
            for (int pc = 0; pc < K4[2]; ++pc)
                for (int pd = 0; pd < K4[3]; ++pd) {
                    real a = al[0][pa], b = al[1][pb], c = al[2][pc], d = al[3][pd];
                    real zeta = a + b, eta = c + d, rho = zeta * eta / (zeta + eta);
                    /* P - A = beta (B - A)/zeta, P - B = alpha (A - B)/zeta (likewise for Q),
                       P - Q = (P - A) - (Q - C) + (A - C), W - P = eta (Q - P)/(zeta+eta),
                       W - Q = zeta (P - Q)/(zeta+eta): the same quantities as the
                       definitions, formed from coordinate differences so that they
                       vanish exactly for coincident centres. */
                    real PA[3], PB[3], QC[3], QD[3], WP[3], WQ[3], PQ2 = 0;
                    for (int i = 0; i < 3; ++i) {
                        PA[i] = b * ((real)B[i] - A[i]) / zeta;
                        PB[i] = a * ((real)A[i] - B[i]) / zeta;
                        QC[i] = d * ((real)D[i] - C[i]) / eta;
                        QD[i] = c * ((real)C[i] - D[i]) / eta;
                        real PQ = PA[i] - QC[i] + ((real)A[i] - C[i]);
                        WP[i] = -eta * PQ / (zeta + eta);
                        WQ[i] = zeta * PQ / (zeta + eta);
                        PQ2 += PQ * PQ;
                    }
                    real T = rho * PQ2;
                    real pref = 2.0 * R_POW(R_PI, (real)2.5) / (zeta * eta * R_SQRT(zeta + eta)) *
                                R_EXP(-a * b / zeta * AB2) * R_EXP(-c * d / eta * CD2);
                    boys_r(Lt, T, F);
                    real i2z = 0.5 / zeta, i2e = 0.5 / eta, i2ze = 0.5 / (zeta + eta);
                    real roz = rho / zeta, roe = rho / eta;

                    for (int ia = 0; ia < w->ta.n; ++ia)
                        for (int ib = 0; ib < w->tb.n; ++ib)
                            for (int ic = 0; ic < w->tc.n; ++ic)
                                for (int id = 0; id < w->td.n; ++id) {
                                    const int *ea = w->ta.t[ia], *eb = w->tb.t[ib];
                                    const int *ec = w->tc.t[ic], *ed = w->td.t[id];
                                    int tot = ea[0] + ea[1] + ea[2] + eb[0] + eb[1] + eb[2] +
                                              ec[0] + ec[1] + ec[2] + ed[0] + ed[1] + ed[2];
                                    int mtop = Lt - tot;
                                    real *v = V + vidx(w, ia, ib, ic, id, 0, M1);
                                    if (tot == 0) {
                                        for (int m = 0; m <= mtop; ++m) v[m] = pref * F[m];
                                        continue;
                                    }
                                    int which, ax = 0;
                                    const int *e;
                                    if (ea[0] + ea[1] + ea[2]) which = 0, e = ea;
                                    else if (eb[0] + eb[1] + eb[2]) which = 1, e = eb;
                                    else if (ec[0] + ec[1] + ec[2]) which = 2, e = ec;
                                    else which = 3, e = ed;
                                    while (e[ax] == 0) ++ax;
                                    int a2[3] = {ea[0], ea[1], ea[2]}, b2[3] = {eb[0], eb[1], eb[2]};
                                    int c2[3] = {ec[0], ec[1], ec[2]}, d2[3] = {ed[0], ed[1], ed[2]};
                                    int *lowered = which == 0 ? a2 : which == 1 ? b2 : which == 2 ? c2 : d2;
                                    lowered[ax] -= 1; /* parent state: the reduced index lowered once */
#define IDX_A(x) w->ta.idx[(x)[0]][(x)[1]][(x)[2]]
#define IDX_B(x) w->tb.idx[(x)[0]][(x)[1]][(x)[2]]
#define IDX_C(x) w->tc.idx[(x)[0]][(x)[1]][(x)[2]]
#define IDX_D(x) w->td.idx[(x)[0]][(x)[1]][(x)[2]]
                                    const real *v0 = V + vidx(w, IDX_A(a2), IDX_B(b2), IDX_C(c2), IDX_D(d2), 0, M1);
                                    real g1, g2, two_exp_inv, ratio;
                                    if (which == 0) g1 = PA[ax], g2 = WP[ax], two_exp_inv = i2z, ratio = roz;
                                    else if (which == 1) g1 = (ORACLE_MUTANT == 7 ? PA[ax] : PB[ax]), g2 = WP[ax], two_exp_inv = i2z, ratio = roz;
                                    else if (which == 2) g1 = QC[ax], g2 = WQ[ax], two_exp_inv = i2e, ratio = roe;
                                    else g1 = QD[ax], g2 = WQ[ax], two_exp_inv = i2e, ratio = roe;
                                    if (ORACLE_MUTANT == 2) g2 = -g2;
                                    if (ORACLE_MUTANT == 3 && which < 2) ratio = roe;
                                    for (int m = 0; m <= mtop; ++m) v[m] = g1 * v0[m] + g2 * v0[m + 1];
                                    /* same-side terms: the lowered index and its partner on
                                       the same electron, each lowered again along ax */
                                    for (int s = 0; s < 4; ++s) {
                                        int *x = s == 0 ? a2 : s == 1 ? b2 : s == 2 ? c2 : d2;
                                        int same_side = (which < 2) == (s < 2);
                                        if (x[ax] == 0) continue;
                                        real n = x[ax];
                                        x[ax] -= 1;
                                        const real *vp = V + vidx(w, IDX_A(a2), IDX_B(b2), IDX_C(c2), IDX_D(d2), 0, M1);
                                        x[ax] += 1;
                                        if (same_side) {
                                            for (int m = 0; m <= mtop; ++m)
                                                v[m] += n * two_exp_inv * (vp[m] - ratio * vp[m + 1]);
                                        } else if (ORACLE_MUTANT != 1) {
                                            for (int m = 0; m <= mtop; ++m) v[m] += n * i2ze * vp[m + 1];
                                        }
                                    }
                                }
                    /* contract the m = 0 entries with the exact target totals */
                    real cw = cc[0][pa] * cc[1][pb] * cc[2][pc] * cc[3][pd];
                    size_t o = 0;
                    if (!dout) {
                        for (int qa = 0; qa < na; ++qa)
                            for (int qb = 0; qb < nb; ++qb)
                                for (int qc = 0; qc < nc; ++qc)
                                    for (int qd = 0; qd < nd; ++qd, ++o) {
                                        size_t k = vidx(w, IDX_A(ca[qa]), IDX_B(cb[qb]), IDX_C(ccc[qc]), IDX_D(cd[qd]), 0, M1);
                                        out[o] += cw * V[k];
                                    }
                        continue;
                    }
                    const real ex4[4] = {a, b, c, d};
                    for (int qa = 0; qa < na; ++qa)
                        for (int qb = 0; qb < nb; ++qb)
                            for (int qc = 0; qc < nc; ++qc)
                                for (int qd = 0; qd < nd; ++qd, ++o) {
                                    for (int p = 0; p < 4; ++p)
                                        for (int i = 0; i < 3; ++i) {
                                            int t4[4][3] = {{ca[qa][0], ca[qa][1], ca[qa][2]}, {cb[qb][0], cb[qb][1], cb[qb][2]},
                                                            {ccc[qc][0], ccc[qc][1], ccc[qc][2]}, {cd[qd][0], cd[qd][1], cd[qd][2]}};
                                            int n = t4[p][i];
                                            t4[p][i] += 1;
                                            real up = V[vidx(w, IDX_A(t4[0]), IDX_B(t4[1]), IDX_C(t4[2]), IDX_D(t4[3]), 0, M1)];
                                            real dn = 0.0;
                                            if (n > 0) {
                                                t4[p][i] -= 2;
                                                dn = V[vidx(w, IDX_A(t4[0]), IDX_B(t4[1]), IDX_C(t4[2]), IDX_D(t4[3]), 0, M1)];
                                            }
                                            dout[(size_t)(3 * p + i) * nout + o] += cw * ((ORACLE_MUTANT == 9 ? 1.0 : 2.0) * ex4[p] * up - n * dn);
                                        }
                                }
                }
}

/* Apply T^(l) to index `pos` (0..3) of a 4-index tensor with dims n[4]:
 * out = (... x T x ...) in, changing dimension n[pos] from ncart to nsph. */
static void transform_index(const real *in, real *out, int n[4], int pos, const real *T, int nsp)
{
    int before = 1, after = 1;
    for (int i = 0; i < pos; ++i) before *= n[i];
    for (int i = pos + 1; i < 4; ++i) after *= n[i];
    int nc = n[pos];
    for (int x = 0; x < before; ++x)
        for (int s = 0; s < nsp; ++s)
            for (int y = 0; y < after; ++y) {
                real acc = 0.0;
                for (int c = 0; c < nc; ++c) acc += T[s * nc + c] * in[((size_t)x * nc + c) * after + y];
                out[((size_t)x * nsp + s) * after + y] = acc;
            }
    n[pos] = nsp;
}

/* ------------------------------------------------------------------------ */
/* Batch entry point                                                         */
/* ------------------------------------------------------------------------ */
/* quartets[nq*4] shell indices in the order to be evaluated; out_off[nq]
 * offsets (in doubles) of each block in `out`; block layout row-major over
 * (a, b, c, d) with Cartesian or spherical components per `flags`.          */
int oracle_eri_quartets(int nshell, const double *centers, const int32_t *l, const int32_t *nprim,
                        const int32_t *prim_off, const double *exps, const double *coefs, int flags,
                        int64_t nq, const int32_t *quartets, const int64_t *out_off, double *out)
{
    for (int s = 0; s < nshell; ++s)
        if (l[s] < 0 || l[s] > OR_LMAX || nprim[s] < 1) return -1;
    /* normalised coefficients */
    int ntot = prim_off[nshell];
    real *cn = (real *)malloc(sizeof(real) * (ntot > 0 ? ntot : 1));
    for (int s = 0; s < nshell; ++s) {
        if (flags & OR_NO_NORMALIZE)
            for (int k = 0; k < nprim[s]; ++k) cn[prim_off[s] + k] = coefs[prim_off[s] + k];
        else
            normalize_r(l[s], nprim[s], exps + prim_off[s], coefs + prim_off[s], cn + prim_off[s]);
    }
    real Tsph[OR_LMAX + 1][(2 * OR_LMAX + 1) * OR_NCART];
    for (int L = 0; L <= OR_LMAX; ++L) sph_coeffs_r(L, Tsph[L]);
    int bad = 0;
#pragma omp parallel
    {
        os_work *w = (os_work *)calloc(1, sizeof(os_work));
        real *buf1 = NULL, *buf2 = NULL;
        size_t bcap = 0;
#pragma omp for schedule(dynamic, 1)
        for (int64_t q = 0; q < nq; ++q) {
            int sh[4], l4[4], K4[4];
            const double *cen[4], *al[4];
            const real *cc[4];
            int ok = 1;
            for (int t = 0; t < 4; ++t) {
                sh[t] = quartets[4 * q + t];
                if (sh[t] < 0 || sh[t] >= nshell) ok = 0;
            }
            if (!ok) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            for (int t = 0; t < 4; ++t) {
                l4[t] = l[sh[t]];
                K4[t] = nprim[sh[t]];
                cen[t] = centers + 3 * sh[t];
                al[t] = exps + prim_off[sh[t]];
                cc[t] = cn + prim_off[sh[t]];
            }
            size_t ncar = (size_t)ncart(l4[0]) * ncart(l4[1]) * ncart(l4[2]) * ncart(l4[3]);
            if (ncar > bcap) {
                free(buf1);
                free(buf2);
                buf1 = (real *)malloc(ncar * sizeof(real));
                buf2 = (real *)malloc(ncar * sizeof(real));
                bcap = ncar;
            }
            os_quartet(w, l4, cen, K4, al, cc, buf1, NULL);
            real *src = buf1, *dst = buf2;
            int n[4] = {ncart(l4[0]), ncart(l4[1]), ncart(l4[2]), ncart(l4[3])};
            if (flags & OR_SPHERICAL)
                for (int pos = 0; pos < 4; ++pos) {
                    transform_index(src, dst, n, pos, Tsph[l4[pos]], nsph(l4[pos]));
                    real *t = src;
                    src = dst;
                    dst = t;
                }
            size_t nv = (size_t)n[0] * n[1] * n[2] * n[3];
            for (size_t x = 0; x < nv; ++x) out[out_off[q] + x] = (double)src[x];
        }
        free(buf1);
        free(buf2);
        free(w->V);
        free(w);
    }
    free(cn);
    return bad ? -1 : 0;
}

/* First derivatives of each quartet's block with respect to the 12 centre
 * coordinates of its four shells in the order given (A_x A_y A_z B_x ...
 * D_z): out + out_off[q] holds 12 blocks of the quartet's block size, one
 * after another, each row-major over (a, b, c, d), Cartesian or spherical
 * (the transform applied to all four indices of each Cartesian block). */
int oracle_eri_deriv_quartets(int nshell, const double *centers, const int32_t *l, const int32_t *nprim,
                              const int32_t *prim_off, const double *exps, const double *coefs, int flags,
                              int64_t nq, const int32_t *quartets, const int64_t *out_off, double *out)
{
    for (int s = 0; s < nshell; ++s)
        if (l[s] < 0 || l[s] + 1 > OR_LMAX || nprim[s] < 1) return -1;
    int ntot = prim_off[nshell];
    real *cn = (real *)malloc(sizeof(real) * (ntot > 0 ? ntot : 1));
    for (int s = 0; s < nshell; ++s) {
        if (flags & OR_NO_NORMALIZE)
            for (int k = 0; k < nprim[s]; ++k) cn[prim_off[s] + k] = coefs[prim_off[s] + k];
        else
            normalize_r(l[s], nprim[s], exps + prim_off[s], coefs + prim_off[s], cn + prim_off[s]);
    }
    real Tsph[OR_LMAX + 1][(2 * OR_LMAX + 1) * OR_NCART];
    for (int L = 0; L <= OR_LMAX; ++L) sph_coeffs_r(L, Tsph[L]);
    int bad = 0;
#pragma omp parallel
    {
        os_work *w = (os_work *)calloc(1, sizeof(os_work));
        real *buf1 = NULL, *buf2 = NULL, *dbuf = NULL;
        size_t bcap = 0;
#pragma omp for schedule(dynamic, 1)
        for (int64_t q = 0; q < nq; ++q) {
            int sh[4], l4[4], K4[4];
            const double *cen[4], *al[4];
            const real *cc[4];
            int ok = 1;
            for (int t = 0; t < 4; ++t) {
                sh[t] = quartets[4 * q + t];
                if (sh[t] < 0 || sh[t] >= nshell) ok = 0;
            }
            if (!ok) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            for (int t = 0; t < 4; ++t) {
                l4[t] = l[sh[t]];
                K4[t] = nprim[sh[t]];
                cen[t] = centers + 3 * sh[t];
                al[t] = exps + prim_off[sh[t]];
                cc[t] = cn + prim_off[sh[t]];
            }
            size_t ncar = (size_t)ncart(l4[0]) * ncart(l4[1]) * ncart(l4[2]) * ncart(l4[3]);
            if (ncar > bcap) {
                free(buf1);
                free(buf2);
                free(dbuf);
                buf1 = (real *)malloc(ncar * sizeof(real));
                buf2 = (real *)malloc(ncar * sizeof(real));
                dbuf = (real *)malloc(12 * ncar * sizeof(real));
                bcap = ncar;
            }
            os_quartet(w, l4, cen, K4, al, cc, NULL, dbuf);
            if (!(flags & OR_SPHERICAL)) {
                for (size_t x = 0; x < 12 * ncar; ++x) out[out_off[q] + x] = (double)dbuf[x];
                continue;
            }
            size_t nsp = (size_t)nsph(l4[0]) * nsph(l4[1]) * nsph(l4[2]) * nsph(l4[3]);
            for (int k = 0; k < 12; ++k) {
                int n[4] = {ncart(l4[0]), ncart(l4[1]), ncart(l4[2]), ncart(l4[3])};
                memcpy(buf1, dbuf + (size_t)k * ncar, ncar * sizeof(real));
                real *src = buf1, *dst = buf2;
                for (int pos = 0; pos < 4; ++pos) {
                    transform_index(src, dst, n, pos, Tsph[l4[pos]], nsph(l4[pos]));
                    real *t = src;
                    src = dst;
                    dst = t;
                }
                for (size_t x = 0; x < nsp; ++x) out[out_off[q] + (size_t)k * nsp + x] = (double)src[x];
            }
        }
        free(buf1);
        free(buf2);
        free(dbuf);
        free(w->V);
        free(w);
    }
    free(cn);
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Schwarz factors                                                           */
/* ------------------------------------------------------------------------ */
/* Reading (the page has no screening rule): S_ij = max over the (ij|ij)
 * block of |(mu nu|mu nu)|, spherical or Cartesian per `flags`, for every
 * pair i >= j; the pair index is i(i+1)/2 + j.                              */
int oracle_schwarz(int nshell, const double *centers, const int32_t *l, const int32_t *nprim,
                   const int32_t *prim_off, const double *exps, const double *coefs, int flags,
                   double *S)
{
    int64_t np = (int64_t)nshell * (nshell + 1) / 2;
    int32_t *qs = (int32_t *)malloc(sizeof(int32_t) * 4 * np);
    int64_t *off = (int64_t *)malloc(sizeof(int64_t) * np);
    int64_t tot = 0;
    for (int i = 0, p = 0; i < nshell; ++i)
        for (int j = 0; j <= i; ++j, ++p) {
            qs[4 * p] = i;
            qs[4 * p + 1] = j;
            qs[4 * p + 2] = i;
            qs[4 * p + 3] = j;
            off[p] = tot;
            int ni = (flags & OR_SPHERICAL) ? nsph(l[i]) : ncart(l[i]);
            int nj = (flags & OR_SPHERICAL) ? nsph(l[j]) : ncart(l[j]);
            tot += (int64_t)ni * nj * ni * nj;
        }
    double *buf = (double *)malloc(sizeof(double) * (tot > 0 ? tot : 1));
    int rc = oracle_eri_quartets(nshell, centers, l, nprim, prim_off, exps, coefs, flags, np, qs, off, buf);
    for (int i = 0, p = 0; i < nshell; ++i)
        for (int j = 0; j <= i; ++j, ++p) {
            int ni = (flags & OR_SPHERICAL) ? nsph(l[i]) : ncart(l[i]);
            int nj = (flags & OR_SPHERICAL) ? nsph(l[j]) : ncart(l[j]);
            int nij = ni * nj;
            double mx = 0.0;
            for (int u = 0; u < nij; ++u) {
                double v = fabs(buf[off[p] + (int64_t)u * nij + u]);
                if (v > mx) mx = v;
            }
            S[p] = mx;
        }
    free(qs);
    free(off);
    free(buf);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* J from a list of unique quartets                                          */
/* ------------------------------------------------------------------------ */
/* J_mu,nu = sum_(la,si) (mu nu|la si) D_la,si (the J update of Algorithm 2).
 * Reading of the page's 8-fold symmetry taken through weighting factors: for a
 * unique quartet (ij|kl) with integrals I, and D~_kl = D_kl * (2 if k != l
 * else 1) taken per shell pair,
 *   J_ij += I . D~_kl ;  and, if the pairs (ij) and (kl) differ,
 *   J_kl += I^T . D~_ij ;
 * then the (j,i) blocks are filled from the (i,j) blocks.  Blocks are taken
 * in the quartet's own shell order.  bf_off[s] = first basis function of
 * shell s; ints/int_off are the integrals for each quartet as produced by
 * oracle_eri_quartets with the same flags.                                  */
static int pair_key(int i, int j) { return i >= j ? i * (i + 1) / 2 + j : j * (j + 1) / 2 + i; }

void oracle_J_from_quartets(int nshell, const int32_t *l, int flags, const int32_t *bf_off, int nbf,
                            int64_t nq, const int32_t *quartets, const int64_t *int_off,
                            const double *ints, const double *Dm, double *J)
{
    for (int64_t x = 0; x < (int64_t)nbf * nbf; ++x) J[x] = 0.0;
    for (int64_t q = 0; q < nq; ++q) {
        int i = quartets[4 * q], j = quartets[4 * q + 1], k = quartets[4 * q + 2], m = quartets[4 * q + 3];
        int ni = (flags & OR_SPHERICAL) ? nsph(l[i]) : ncart(l[i]);
        int nj = (flags & OR_SPHERICAL) ? nsph(l[j]) : ncart(l[j]);
        int nk = (flags & OR_SPHERICAL) ? nsph(l[k]) : ncart(l[k]);
        int nm = (flags & OR_SPHERICAL) ? nsph(l[m]) : ncart(l[m]);
        const double *I = ints + int_off[q];
        double fkl = (k != m && ORACLE_MUTANT != 8) ? 2.0 : 1.0, fij = (i != j) ? 2.0 : 1.0;
        int same = pair_key(i, j) == pair_key(k, m);
        for (int a = 0; a < ni; ++a)
            for (int b = 0; b < nj; ++b)
                for (int c = 0; c < nk; ++c)
                    for (int d = 0; d < nm; ++d) {
                        double v = I[((a * nj + b) * nk + c) * nm + d];
                        J[(int64_t)(bf_off[i] + a) * nbf + bf_off[j] + b] += fkl * v * Dm[(int64_t)(bf_off[k] + c) * nbf + bf_off[m] + d];
                        if (!same)
                            J[(int64_t)(bf_off[k] + c) * nbf + bf_off[m] + d] += fij * v * Dm[(int64_t)(bf_off[i] + a) * nbf + bf_off[j] + b];
                    }
    }
    /* an off-diagonal shell block may have been accumulated in either
       orientation, depending on each quartet's shell order: add the two
       orientations and store the sum in both (J is symmetric).  Diagonal
       shell blocks are already complete in both (a,b) and (b,a). */
    for (int i = 0; i < nshell; ++i)
        for (int j = 0; j < i; ++j) {
            int ni = (flags & OR_SPHERICAL) ? nsph(l[i]) : ncart(l[i]);
            int nj = (flags & OR_SPHERICAL) ? nsph(l[j]) : ncart(l[j]);
            for (int a = 0; a < ni; ++a)
                for (int b = 0; b < nj; ++b) {
                    int64_t x = (int64_t)(bf_off[i] + a) * nbf + bf_off[j] + b;
                    int64_t y = (int64_t)(bf_off[j] + b) * nbf + bf_off[i] + a;
                    double s = J[x] + J[y];
                    J[x] = s;
                    J[y] = s;
                }
        }
}

/* J_mu,nu by the plain four-index sum over all shell quadruples (no symmetry). */
int oracle_J_naive(int nshell, const double *centers, const int32_t *l, const int32_t *nprim,
                   const int32_t *prim_off, const double *exps, const double *coefs, int flags,
                   const int32_t *bf_off, int nbf, const double *Dm, double *J)
{
    int64_t nq = (int64_t)nshell * nshell * nshell * nshell;
    int32_t *qs = (int32_t *)malloc(sizeof(int32_t) * 4 * nq);
    int64_t *off = (int64_t *)malloc(sizeof(int64_t) * nq);
    int64_t tot = 0, q = 0;
    for (int i = 0; i < nshell; ++i)
        for (int j = 0; j < nshell; ++j)
            for (int k = 0; k < nshell; ++k)
                for (int m = 0; m < nshell; ++m, ++q) {
                    qs[4 * q] = i, qs[4 * q + 1] = j, qs[4 * q + 2] = k, qs[4 * q + 3] = m;
                    off[q] = tot;
                    int n1 = (flags & OR_SPHERICAL) ? nsph(l[i]) : ncart(l[i]);
                    int n2 = (flags & OR_SPHERICAL) ? nsph(l[j]) : ncart(l[j]);
                    int n3 = (flags & OR_SPHERICAL) ? nsph(l[k]) : ncart(l[k]);
                    int n4 = (flags & OR_SPHERICAL) ? nsph(l[m]) : ncart(l[m]);
                    tot += (int64_t)n1 * n2 * n3 * n4;
                }
    double *buf = (double *)malloc(sizeof(double) * tot);
    int rc = oracle_eri_quartets(nshell, centers, l, nprim, prim_off, exps, coefs, flags, nq, qs, off, buf);
    for (int64_t x = 0; x < (int64_t)nbf * nbf; ++x) J[x] = 0.0;
    for (q = 0; q < nq; ++q) {
        int i = qs[4 * q], j = qs[4 * q + 1], k = qs[4 * q + 2], m = qs[4 * q + 3];
        int n1 = (flags & OR_SPHERICAL) ? nsph(l[i]) : ncart(l[i]);
        int n2 = (flags & OR_SPHERICAL) ? nsph(l[j]) : ncart(l[j]);
        int n3 = (flags & OR_SPHERICAL) ? nsph(l[k]) : ncart(l[k]);
        int n4 = (flags & OR_SPHERICAL) ? nsph(l[m]) : ncart(l[m]);
        const double *I = buf + off[q];
        for (int a = 0; a < n1; ++a)
            for (int b = 0; b < n2; ++b)
                for (int c = 0; c < n3; ++c)
                    for (int d = 0; d < n4; ++d)
                        J[(int64_t)(bf_off[i] + a) * nbf + bf_off[j] + b] +=
                            I[((a * n2 + b) * n3 + c) * n4 + d] * Dm[(int64_t)(bf_off[k] + c) * nbf + bf_off[m] + d];
    }
    free(qs);
    free(off);
    free(buf);
    return rc;
}

/* Exchange matrix K_mu,nu = sum_(la,si) (mu la|nu si) D_la,si (the Coulomb
   integrals of Eq. (1) contracted with the density along the second index of
   each electron; no factor -1/2).  Plain four-index sum over every ordered
   shell quadruple, no symmetry (tiny inputs only). */
int oracle_K_naive(int nshell, const double *centers, const int32_t *l, const int32_t *nprim,
                   const int32_t *prim_off, const double *exps, const double *coefs, int flags,
                   const int32_t *bf_off, int nbf, const double *Dm, double *K)
{
    int64_t nq = (int64_t)nshell * nshell * nshell * nshell;
    int32_t *qs = (int32_t *)malloc(sizeof(int32_t) * 4 * nq);
    int64_t *off = (int64_t *)malloc(sizeof(int64_t) * nq);
    int64_t tot = 0, q = 0;
    for (int i = 0; i < nshell; ++i)
        for (int j = 0; j < nshell; ++j)
            for (int k = 0; k < nshell; ++k)
                for (int m = 0; m < nshell; ++m, ++q) {
                    qs[4 * q] = i, qs[4 * q + 1] = j, qs[4 * q + 2] = k, qs[4 * q + 3] = m;
                    off[q] = tot;
                    int n1 = (flags & OR_SPHERICAL) ? nsph(l[i]) : ncart(l[i]);
                    int n2 = (flags & OR_SPHERICAL) ? nsph(l[j]) : ncart(l[j]);
                    int n3 = (flags & OR_SPHERICAL) ? nsph(l[k]) : ncart(l[k]);
                    int n4 = (flags & OR_SPHERICAL) ? nsph(l[m]) : ncart(l[m]);
                    tot += (int64_t)n1 * n2 * n3 * n4;
                }
    double *buf = (double *)malloc(sizeof(double) * tot);
    int rc = oracle_eri_quartets(nshell, centers, l, nprim, prim_off, exps, coefs, flags, nq, qs, off, buf);
    for (int64_t x = 0; x < (int64_t)nbf * nbf; ++x) K[x] = 0.0;
    for (q = 0; q < nq; ++q) {
        int i = qs[4 * q], j = qs[4 * q + 1], k = qs[4 * q + 2], m = qs[4 * q + 3];
        int n1 = (flags & OR_SPHERICAL) ? nsph(l[i]) : ncart(l[i]);
        int n2 = (flags & OR_SPHERICAL) ? nsph(l[j]) : ncart(l[j]);
        int n3 = (flags & OR_SPHERICAL) ? nsph(l[k]) : ncart(l[k]);
        int n4 = (flags & OR_SPHERICAL) ? nsph(l[m]) : ncart(l[m]);
        const double *I = buf + off[q];
        for (int a = 0; a < n1; ++a)
            for (int b = 0; b < n2; ++b)
                for (int c = 0; c < n3; ++c)
                    for (int d = 0; d < n4; ++d)
                        K[(int64_t)(bf_off[i] + a) * nbf + bf_off[k] + c] +=
                            I[((a * n2 + b) * n3 + c) * n4 + d] * Dm[(int64_t)(bf_off[j] + b) * nbf + bf_off[m] + d];
    }
    free(qs);
    free(off);
    free(buf);
    return rc;
}

/* K from unique quartets: every distinct ordered shell quadruple among the
   eight index permutations of a unique quartet (ij|kl) = (ji|kl) = (ij|lk) =
   (kl|ij) = ... is added once, with the block element taken from the unique
   quartet's block by the corresponding index permutation. */
void oracle_K_from_quartets(int nshell, const int32_t *l, int flags, const int32_t *bf_off, int nbf,
                            int64_t nq, const int32_t *quartets, const int64_t *int_off,
                            const double *ints, const double *Dm, double *K)
{
    (void)nshell;
    for (int64_t x = 0; x < (int64_t)nbf * nbf; ++x) K[x] = 0.0;
    for (int64_t q = 0; q < nq; ++q) {
        const int s[4] = {quartets[4 * q], quartets[4 * q + 1], quartets[4 * q + 2], quartets[4 * q + 3]};
        int n[4];
        for (int t = 0; t < 4; ++t) n[t] = (flags & OR_SPHERICAL) ? nsph(l[s[t]]) : ncart(l[s[t]]);
        const double *I = ints + int_off[q];
        /* the eight permutations as positions of the unique quartet's indices */
        static const int perms[8][4] = {{0, 1, 2, 3}, {1, 0, 2, 3}, {0, 1, 3, 2}, {1, 0, 3, 2},
                                        {2, 3, 0, 1}, {3, 2, 0, 1}, {2, 3, 1, 0}, {3, 2, 1, 0}};
        int seen[8][4], nseen = 0;
        for (int p = 0; p < 8; ++p) {
            int t4[4];
            for (int t = 0; t < 4; ++t) t4[t] = s[perms[p][t]];
            int dup = 0;
            for (int u = 0; u < nseen; ++u)
                if (seen[u][0] == t4[0] && seen[u][1] == t4[1] && seen[u][2] == t4[2] && seen[u][3] == t4[3]) dup = 1;
            if (dup) continue;
            for (int t = 0; t < 4; ++t) seen[nseen][t] = t4[t];
            ++nseen;
            /* element (x0 x1|x2 x3) of the permuted quartet = I at the unique quartet's
               positions: index x_t belongs to position perms[p][t] */
            int x[4];
            for (x[0] = 0; x[0] < n[perms[p][0]]; ++x[0])
                for (x[1] = 0; x[1] < n[perms[p][1]]; ++x[1])
                    for (x[2] = 0; x[2] < n[perms[p][2]]; ++x[2])
                        for (x[3] = 0; x[3] < n[perms[p][3]]; ++x[3]) {
                            int y[4];
                            for (int t = 0; t < 4; ++t) y[perms[p][t]] = x[t];
                            double v = I[((y[0] * n[1] + y[1]) * n[2] + y[2]) * n[3] + y[3]];
                            K[(int64_t)(bf_off[t4[0]] + x[0]) * nbf + bf_off[t4[2]] + x[2]] +=
                                v * Dm[(int64_t)(bf_off[t4[1]] + x[1]) * nbf + bf_off[t4[3]] + x[3]];
                        }
        }
    }
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
