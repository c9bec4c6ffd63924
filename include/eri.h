/*
 * eri.h -- C ABI of the MI355X (gfx950) four-centre ERI engine.
 *
 * What is computed (source: "FusionRCG: Orchestrating Recursive Computation
 * Graphs across GPU Memory Hierarchies", Wei et al.):
 *   - contracted electron repulsion integrals (ab|cd) over Cartesian Gaussian
 *     shells, Eq. (1) of section II-A, evaluated by the two-phase recurrence of
 *     section II-A (vertical recurrence Eq. (2) from Boys values, contraction
 *     over primitive quartets as in Algorithm 2 of section III-C, horizontal
 *     recurrence Eq. (3));
 *   - optionally in the real spherical basis, Eq. (8) of section III-B, with
 *     the transform applied index by index inside the horizontal phase
 *     (stepwise fusion, Eqs. (11)-(16), identical to Eq. (17));
 *   - the Coulomb matrix J_mu,nu = sum_(la,si) (mu nu|la si) D_la,si that
 *     Algorithm 2 accumulates from each quartet, using the 8-fold permutation symmetry of
 *     section III-C2 (Kernel 2) over Schwarz-screened unique quartets, and the
 *     exchange matrix K it scatters beside J.
 *
 * Conventions (not fixed by the page; chosen and documented here):
 *   - Cartesian components of a shell with angular momentum l are ordered
 *     x-power descending, then y-power descending (d: xx xy xz yy yz zz).
 *   - Every Cartesian component of a primitive carries the factor
 *     N(alpha,l) = (2 alpha/pi)^(3/4) (4 alpha)^(l/2) / sqrt((2l-1)!!); the
 *     contracted x^l component is then scaled to unit norm.  ERI_NO_NORMALIZE
 *     uses the raw coefficients on raw monomials instead.
 *   - Spherical components are real solid harmonics without Condon-Shortley
 *     phase, m = -l..l (a p shell comes out as y, z, x), orthonormal for the
 *     normalised shell, leading monomial positive.
 *   - A block (ab|cd) is stored row-major over (a, b, c, d).
 *   - Basis functions of the J/D matrices are numbered shell by shell in the
 *     order of the shell arrays, components contiguous within a shell.
 *   - Quartet classes: pair class pc(la,lb) = la(la+1)/2 + lb (la >= lb),
 *     class id = pcb(pcb+1)/2 + pck with pcb >= pck; 120 classes for l <= 4.
 *   - Canonical quartet: swap a<->b if l_a < l_b (bit 0 of perm), c<->d if
 *     l_c < l_d (bit 1), then bra<->ket if pc(bra) < pc(ket) (bit 2).  Blocks
 *     are produced for the canonical quartet; the index map records it.
 *
 * Memory.  The caller owns all device memory; the library allocates none.
 * Every call that needs device work memory takes a workspace: called with
 * workspace == NULL it writes the bytes it needs to *ws_bytes and does nothing
 * else; called with a workspace (256-byte aligned) of *ws_bytes bytes it
 * works inside it (ERI_E_WORKSPACE if *ws_bytes is below the size the query
 * returned).  A plan's device data live in the workspace given to
 * eri_build_quartets, which must stay allocated and untouched until
 * eri_plan_destroy; the other workspaces are free again when the call's work
 * on `stream` has finished.  The library's only device memory of its own are
 * two file-scope arrays per device: the Boys-function table (221 KB, written
 * once per device by the first plan build there) and the FMA-rate sink.
 * Host pointers are marked "(host)", device pointers "(device)".
 *
 * Streams.  All device work is enqueued on `stream` (a hipStream_t, NULL =
 * default stream) and on the side streams the caller registered with
 * eri_plan_set_streams; the library creates no stream.  Calls that must return
 * a count computed on the device synchronise `stream` and say so.  Calls on
 * one plan must not overlap in time (they share the plan's scratch and chunk
 * lists).
 *
 * Errors.  Every function returns ERI_OK or a negative code and never throws;
 * arguments are validated before anything is launched.  Results are
 * deterministic: the same inputs on the same device give bitwise-identical
 * outputs (no floating-point atomics).
 */
#ifndef ERI_MI355X_H
#define ERI_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ERI_OK 0
#define ERI_E_INVALID (-1)     /* malformed argument (index out of range, l > 4, K < 1, ...) */
#define ERI_E_UNSUPPORTED (-2) /* valid request the library does not implement */
#define ERI_E_CAPACITY (-3)    /* output buffer smaller than the call's output */
#define ERI_E_HIP (-4)         /* a HIP runtime call failed; see eri_strerror */
#define ERI_E_NOMEM (-5)       /* host memory exhausted */
#define ERI_E_WORKSPACE (-6)   /* workspace smaller than the size query returned */

#define ERI_SPHERICAL 1    /* output in the real spherical basis */
#define ERI_NO_NORMALIZE 2 /* raw coefficients on raw monomials */

#define ERI_MAX_L 4
#define ERI_MAX_PRIM 15
#define ERI_MAX_SIDE_STREAMS 3

/* Shells as structure-of-arrays, all host memory, read (and copied) during
 * eri_build_quartets only.  The page's statement of the problem (section
 * III-C, the input of Algorithm 2): each shell has a centre, an angular momentum and
 * primitives {(alpha_i, c_i)}. */
typedef struct eri_shells {
    int32_t nshell;
    const double *centers;   /* [3*nshell], bohr */
    const int32_t *l;        /* [nshell], 0..ERI_MAX_L */
    const int32_t *nprim;    /* [nshell], 1..ERI_MAX_PRIM */
    const int32_t *prim_off; /* [nshell+1], CSR offsets into exps/coefs, prim_off[0] = 0 */
    const double *exps;      /* [prim_off[nshell]], > 0 */
    const double *coefs;     /* [prim_off[nshell]], raw contraction coefficients */
} eri_shells;

typedef struct eri_plan eri_plan;

/*
 * Build a quartet plan: the shells' primitive-pair data (the Gaussian-pair step
 * of Algorithm 2), and the quartets batched by angular-momentum class and
 * contraction length (section III-C: kernels per shell-quartet class; the 120
 * classes of section IV for l <= 4).
 *   quartets != NULL (host): explicit list of nq shell quartets [4*nq]; each
 *     is canonicalised and the list ordered by (class id, K_a K_b, K_c K_d,
 *     input position).  tau must be 0.
 *   quartets == NULL: all unique quartets (pair(ij) >= pair(kl), i >= j,
 *     k >= l) that pass the Schwarz test fl(S_ij * S_kl) >= fl(tau * tau),
 *     with S_ij = max |(mu nu|mu nu)| over the (ij|ij) block, computed on the
 *     device by the same class kernels as sums over sub-pair quartets of at
 *     most 6 primitive pairs per side (tau = 0 keeps every quartet; the page
 *     states no screen, this is the reading taken).  Such plans keep only the
 *     primitive pairs (alpha, beta) of a shell pair with
 *     alpha beta / (alpha + beta) |AB|^2 <= 230 (their Gaussian-product factor
 *     is at least 1.3e-100; a shell pair with none keeps its first), and
 *     K_pair counts those.  Pairs are bucketed
 *     by (pair class, K_pair) and ranked by S descending (ties by pair index);
 *     order (class id, K_bra, K_ket, bra rank, ket rank).  Because the kets of
 *     one bra are ranked by S descending, the survivors of each (block, bra)
 *     are a prefix of its ket list: the plan stores only these prefix lengths
 *     and their running offsets (memory per (bucket pair, bra pair), not per
 *     quartet) and expands slot lists on the device in chunks of at most
 *     ERI_CHUNK_QUARTETS (an environment variable read here, default 4194304).
 *   workspace == NULL: *ws_bytes <- bytes the plan needs (host arithmetic
 *     and hipCUB's temp-storage size queries, which read the current device's
 *     properties; no device work, no synchronisation); *plan is not written.
 *   workspace != NULL (device, 256-byte aligned, *ws_bytes bytes): the plan
 *     is built inside it and *plan receives the plan.  Synchronises `stream`
 *     (class-block sizes are needed on the host).
 * Errors: ERI_E_INVALID for malformed shells, flags or quartets (validated on
 * the host before any launch), ERI_E_WORKSPACE, ERI_E_UNSUPPORTED for more
 * than 2^30 listed quartets or 2^30 shell pairs.
 */
int eri_build_quartets(const eri_shells *shells, int flags, const int32_t *quartets, int64_t nq, double tau,
                       void *workspace, size_t *ws_bytes, void *stream, eri_plan **plan);

/* Free a plan's host state (NULL is allowed); its workspace is the caller's. */
int eri_plan_destroy(eri_plan *plan);

/* Register up to ERI_MAX_SIDE_STREAMS caller-created streams (hipStream_t,
 * default priority) on which multi-block calls of this plan may run class
 * blocks and digestion chunks concurrently with `stream` (section III-C:
 * the class kernels are independent launches); n = 0 removes them.  The
 * streams must outlive their use by the plan.  Digestion workspaces are sized
 * for the number of streams registered when the size is queried. */
int eri_plan_set_streams(eri_plan *plan, void *const *streams, int32_t n);

/* Sizes (host outputs): quartets, output doubles of all blocks, number of
 * class blocks, basis functions (spherical or Cartesian per the plan's flags),
 * shell pairs. */
int eri_plan_info(const eri_plan *plan, int64_t *n_quartets, int64_t *n_out_doubles, int32_t *n_blocks,
                  int32_t *nbf, int64_t *n_pairs);

/* Per class block b (host arrays of n_blocks): class id, first plan slot,
 * number of quartets, offset (doubles) of its first block in the output. */
int eri_plan_blocks(const eri_plan *plan, int32_t *class_id, int64_t *start, int64_t *count, int64_t *out_offset);

/* Index map of the plan: dst[5*slot + 0..3] = shells (a, b, c, d) of the
 * canonical quartet computed in that slot, dst[5*slot + 4] = perm bits.  dst
 * is device memory [5*n_quartets] (n_quartets < 2^31); asynchronous. */
int eri_plan_index_map(const eri_plan *plan, int32_t *dst, void *stream);

/* The index-map rows of plan slots [first, first + count) only: dst is device
 * memory [5*count], count < 2^31; asynchronous. */
int eri_plan_quartets(const eri_plan *plan, int64_t first, int64_t count, int32_t *dst, void *stream);

/* Schwarz factors S[pair] for pair index i(i+1)/2 + j (screened plans only);
 * dst is device memory [n_pairs]; asynchronous. */
int eri_plan_schwarz(const eri_plan *plan, double *dst, void *stream);

/*
 * Integrals (Eq. (1) by Eqs. (2)-(3), spherical by Eq. (8) fused stepwise,
 * the primitive loop of Algorithm 2) of class blocks [block_begin, block_end) into `out`
 * (device): block b's quartets start at out + out_offset[b] -
 * out_offset[block_begin]; out_capacity is the number of doubles at `out`
 * (ERI_E_CAPACITY if too few).  Work memory is the plan's.  Asynchronous: the
 * blocks run on `stream` and the registered side streams, and `stream` waits
 * for them before later work on it starts.
 */
int eri_compute_batch(const eri_plan *plan, int32_t block_begin, int32_t block_end, double *out,
                      int64_t out_capacity, void *stream);

/*
 * Integrals (as eri_compute_batch) of quartets [first, first + count) of class
 * block `block` (counted from the block's first slot) into `out` (device), one
 * block of outputs per quartet in plan order; out_capacity >= count x (block
 * size) doubles.  For sampling blocks whose full output would not fit.
 * Asynchronous, on `stream` only.
 */
int eri_compute_range(const eri_plan *plan, int32_t block, int64_t first, int64_t count, double *out,
                      int64_t out_capacity, void *stream);

/*
 * Coulomb matrix of a screened plan (the J update of Algorithm 2;
 * section III-C2 Kernel 2, 8-fold symmetry through scale factors):
 * J = sum over the plan's unique quartets with D~_kl = D_kl (2 for k != l),
 * D and J dense row-major device matrices of order nbf with leading dimensions
 * ldd, ldj; D must be symmetric; J is fully overwritten.  Chunk by chunk:
 * integrals, per-quartet contribution vectors, entries sorted by target pair
 * and each pair's run added in an order fixed by the plan, so J is
 * deterministic (no atomics).  Chunks are spread over `stream` and the
 * registered side streams, each with its own chunk buffers and accumulators.
 * workspace == NULL: *ws_bytes <- bytes needed (D and J may be NULL then).
 * Otherwise the call works in the workspace and is asynchronous.
 */
int eri_digest_J(const eri_plan *plan, const double *D, int32_t ldd, double *J, int32_t ldj, void *workspace,
                 size_t *ws_bytes, void *stream);

/*
 * The Coulomb contributions of quartets [first, first + count) of class block
 * `block` of a screened plan (counted from the block's first slot, as
 * eri_compute_range) added to J: the J update of Algorithm 2 restricted to
 * those quartets, with eri_digest_J's D~ weights and row-major layouts.  J is
 * not cleared: over ranges that partition every block, with J zeroed first,
 * the calls add up to eri_digest_J's result (equal to rounding: the chunks are
 * spread over the stream lanes per call).  For J builds longer than one call
 * may take (time-sliced or checkpointed jobs).  ERI_E_INVALID for a block or
 * slot range outside the plan.  Workspace and query as eri_digest_J (a
 * workspace sized for eri_digest_J serves every range); asynchronous.
 */
int eri_digest_J_range(const eri_plan *plan, int32_t block, int64_t first, int64_t count, const double *D,
                       int32_t ldd, double *J, int32_t ldj, void *workspace, size_t *ws_bytes, void *stream);

/*
 * Coulomb and exchange matrices of a screened plan in one pass over its
 * integrals (Algorithm 2 updates J and K from each quartet; section III-C2): J as
 * eri_digest_J, and K_mu,nu = sum (mu la|nu si) D_la,si (no factor -1/2),
 * both over the plan's unique quartets with their index permutations, D
 * symmetric.  J or K may be NULL (not both; the query must pass the same
 * choice as the call); each given matrix (order nbf, leading dimension ldj /
 * ldk, device) is fully overwritten.  K: for a quartet (ij|kl) the four blocks
 * (ik), (jk), (il), (jl), each contracted with D over the other pair of
 * indices, sorted by target block and added in an order fixed by the plan,
 * then K = A + A^T; deterministic.  Workspace as eri_digest_J.
 */
int eri_digest_JK(const eri_plan *plan, const double *D, int32_t ldd, double *J, int32_t ldj, double *K,
                  int32_t ldk, void *workspace, size_t *ws_bytes, void *stream);

/*
 * eri_digest_J without any allocation, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid it).  Same arguments, result and determinism as eri_digest_J,
 * with one stream lane; its chunk buffers live in a file-scope device array of
 * ERI_NOALLOC_SCRATCH_BYTES that each device holds until the process ends, so
 * chunks are smaller (the sums are in another order than eri_digest_J's, equal
 * to rounding).  Nothing of the array needs to start at zero.  Every call on a
 * device shares that device's array: calls that overlap in time on one device
 * race.  ERI_E_WORKSPACE if one quartet of the plan's largest class block does
 * not fit the array; ERI_E_INVALID if the current device is not the plan's.
 * Asynchronous.
 */
#define ERI_NOALLOC_SCRATCH_BYTES (((size_t)64) << 20)
int eri_digest_J_noalloc(const eri_plan *plan, const double *D, int32_t ldd, double *J, int32_t ldj, void *stream);

/*
 * First derivatives of the integrals of plan slots [first, first + count)
 * with respect to the 12 centre coordinates of each canonical quartet (the
 * shells a, b, c, d of the index map): Eq. (1) of section II-A differentiated
 * with respect to the centres; the page's library generates "first-derivative
 * variants" of its class kernels (section IV, build system).  A primitive
 * Cartesian Gaussian differentiated with respect to its own centre gives
 * 2 alpha phi_(a+1_i) - a_i phi_(a-1_i), so each derivative block combines
 * integrals of the two neighbouring classes, which the same class kernels
 * compute on an auxiliary shell set (every shell raised and lowered) planned
 * inside the workspace.
 *   out (device): for every slot, 12 blocks of the slot's block size in the
 *     order d/dA_x, d/dA_y, d/dA_z, d/dB_x, ..., d/dD_z, each row-major over
 *     (a, b, c, d) and Cartesian or spherical per the plan; the slots one
 *     after another, so slot s starts at 12 x (sum of the block sizes of the
 *     slots before it in the range).
 *   out_capacity: doubles available at out (ERI_E_CAPACITY if too few).
 *   count <= 2^24.  Shells up to l = ERI_MAX_L: the library holds the
 *     classes with one shell raised to l = ERI_MAX_L + 1 (Cartesian kernels);
 *     a build without one of the auxiliary classes a range needs (the
 *     ablation variants) returns ERI_E_UNSUPPORTED.
 *   workspace == NULL: *ws_bytes <- bytes needed (out may be NULL then).
 * Both the query and the call read the range's shells back to the host and
 * synchronise `stream`.
 */
int eri_compute_deriv(const eri_plan *plan, int64_t first, int64_t count, double *out, int64_t out_capacity,
                      void *workspace, size_t *ws_bytes, void *stream);

/* Static text for an error code, with the last HIP error for ERI_E_HIP. */
const char *eri_strerror(int code);

/* Measured FP64 FMA rate of the current device in TFLOP/s (host output):
 * the denominator the class kernels' FP64 fraction can also be read against,
 * beside the published peak.  Runs on `stream` and synchronises it. */
int eri_fp64_fma_tflops(double *tflops, void *stream);

/* Class metadata (host outputs): l of (a, b, c, d) and the tier of the
 * class's spherical-output kernels ('V' register tiers, 'M' memory tier); the
 * tier is chosen per output kind (section III-C: multi-tier routing). */
int eri_class_info(int32_t class_id, int32_t *l4, int32_t *tier);

#ifdef __cplusplus
}
#endif

#endif
