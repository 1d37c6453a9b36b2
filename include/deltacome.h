/*
 * deltacome.h -- C ABI of libdeltacome.so: the Delta-CoMe mixed-precision
 * low-rank delta apply on AMD Instinct MI355X (gfx950).
 *
 * What it computes.  A fine-tuned model is served as its backbone W_base plus
 * a compressed delta.  The delta is decomposed by SVD into singular pairs
 * (u_i, sigma_i, v_i); pairs with larger singular values keep more bits: a
 * first group at 8 bits, the next at 3 bits, the next at 2 bits, the rest
 * dropped (0 bits).  Many such deltas share one bf16 backbone.  For a token x
 * served by tenant k:
 *
 *     y = W_base x + U_k diag(sigma_k) (V_k x)        (bf16 out, fp32 sums)
 *
 * Sources (web pages, cited by title and section):
 *   [P1] "Delta-CoMe - 清华联合OpenBMB等高校开源的新型增量压缩算法" (paooo.com):
 *        "Delta-CoMe的技术原理" (low-rank decomposition of the delta by SVD;
 *        mixed-precision bits per singular vector, larger singular values at
 *        higher precision; long-tail spectrum) and "Delta-CoMe的应用场景"
 *        (multi-tenant serving of many fine-tuned models).
 *   [P2] "Delta-CoMe: Training-Free Delta-Compression with Mixed-Precision for
 *        Large Language Models" (atlas.scime.ai summary): "Approach" (8/3/2
 *        bits for successive groups, smallest dropped at 0 bits, same size as
 *        BitDelta at 1/16), "Key results" (a GPU kernel for the apply; 50
 *        models served on one GPU), "Problem" (delta = fine-tuned minus
 *        backbone).
 *   [P4] "Enhancing Delta Compression in LLMs via SVD-based Quantization
 *        Error Minimization" (gist.science): §2.1 (W = U Sigma V, V quantized
 *        row by row).
 *
 * Storage format.  The pages fix no layout.  This library fixes one: b-bit
 * codes packed little-endian into uint32 words (3-bit codes 32 per 3 words)
 * and, for each group of 128 consecutive elements of a singular vector, an
 * fp16 scale s and an fp16 zero z from asymmetric round-to-nearest min/max
 * quantization; the dequantized value of code q is fp16(s * (q - z)).
 *
 * One packed buffer = one tenant's delta for one matrix, spec
 * (out, in, n8, n3, n2); r = n8+n3+n2; Gi = in/128; Go = out/128.  Ranks are
 * numbered 0..r-1: the 8-bit segment, then the 3-bit, then the 2-bit one;
 * "local rank" is the index inside a segment of n = n_b ranks.
 * Bitstream rule: codes c_0, c_1, ... at b bits occupy bits [b*k, b*k+b) of
 * a stream of uint32 words, bit t of the stream being bit t%32 of word t/32.
 * Regions, each at a multiple of 256 bytes from the buffer start, in order:
 *   SIGMA  fp32 [r]
 *   VC_8   V codes at 8 bits, [n][Gi][32] words: the group's 128 codes of
 *          v_i form one bitstream (plain bytes [n][in]).
 *   VC_b   b = 3,2: V codes in 16-rank tiles, [ceil(n/16)][Gi][4][16][b]
 *          words: word block (T, g, q, c) is the bitstream of codes
 *          32q..32q+31 of group g of local rank 16T+c (ranks past n are 0),
 *          so the 16 ranks of a tile lie side by side for each 32-code chunk.
 *   VS_b   V scale/zero, uint32 [Gi][pad4(n)]: fp16 scale | fp16 zero << 16.
 *   UC_8   U codes at 8 bits, bytes [out][n8], byte (o,i) = code of u_i at
 *          row o.
 *   UC_b   b = 3,2: U codes packed along the rank axis.  Ranks are cut into
 *          K-blocks of 32 (KB = ceil(n/32)); K-block kb of row o is the
 *          bitstream of the codes of u_{32kb}..u_{32kb+31} at row o (codes
 *          past n are 0), b words long, except the last K-block, which keeps
 *          wl = ceil(m*b/32) words for its m = n-32(KB-1) ranks.  Rows go in
 *          16-row tiles; a tile is [KB-1][16][b] words then [16][wl] words
 *          (the 16 rows of one K-block contiguous).
 *   US_b   U scale/zero, uint32 [Go][pad4(n)]; entry (g,i) covers rows
 *          128g..128g+127 of u_i.
 * Pad entries are zero.  Total size rounded up to 256 bytes.
 *
 * Conventions for every call.
 *   - Every argument is checked on the host before anything is enqueued; a
 *     call that returns an error has enqueued nothing and written nothing.
 *   - Device calls are asynchronous on `stream` (a hipStream_t passed as
 *     void*; NULL = the null stream) and never synchronize; device faults show
 *     at the caller's next synchronization.
 *   - The caller owns every buffer.  The library allocates no device memory
 *     and keeps no mutable global state; calls on different streams with
 *     different workspaces may run concurrently.  Two calls that share a
 *     workspace must be ordered by the caller.
 *   - bf16 and fp16 tensors are passed as uint16_t bit patterns, row-major.
 *   - Device pointers must be 16-byte aligned (DC_ERR_ALIGN), the workspace
 *     256-byte aligned.
 */
#ifndef DELTACOME_H
#define DELTACOME_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t dc_status;
enum {
  DC_OK = 0,
  DC_ERR_INVALID_ARG = -1, /* null pointer, overlap of x and y, n/T out of range */
  DC_ERR_SHAPE = -2,       /* out/in not a positive multiple of 128, negative
                              counts, r > min(out,in), tenants of one call with
                              different out/in */
  DC_ERR_ALIGN = -3,       /* device pointer not 16-B aligned (workspace 256-B) */
  DC_ERR_BUFFER = -4,      /* buffer or workspace smaller than required */
  DC_ERR_RANGE = -5,       /* dc_pack: non-finite input or fp16 scale overflow */
  DC_ERR_HIP = -6,         /* a HIP launch or query failed */
  DC_ERR_UNSUPPORTED = -7  /* a limit of this build: more than DC_MAX_TENANTS tenants, or a
                              packed buffer, t (T x widest rank row, fp32) or the backbone
                              product (T x out, fp32) of 2 GiB or more */
};

/* Most tenants one multi-tenant or prefill call can address. */
#define DC_MAX_TENANTS 128
/* Most matrices one grouped call (dc_apply_multitenant_group) can take. */
#define DC_MAX_GROUP 4

typedef struct dc_spec {
  int32_t out; /* rows of the matrix (output features), multiple of 128 */
  int32_t in;  /* columns (input features), multiple of 128 */
  int32_t n8;  /* pairs stored at 8 bits (largest singular values) */
  int32_t n3;  /* next pairs, at 3 bits */
  int32_t n2;  /* next pairs, at 2 bits; all later pairs are dropped */
} dc_spec;

/* A packed delta in device memory: the spec and the buffer's first byte.
 * Built by pointer arithmetic only (no copy). */
typedef struct dc_delta_view {
  dc_spec spec;
  const void* base; /* device pointer to dc_packed_bytes(&spec) bytes */
} dc_delta_view;

/* Region ids for dc_region, in storage order. */
enum {
  DC_REG_SIGMA = 0,
  DC_REG_VC8, DC_REG_VC3, DC_REG_VC2,
  DC_REG_VS8, DC_REG_VS3, DC_REG_VS2,
  DC_REG_UC8, DC_REG_UC3, DC_REG_UC2,
  DC_REG_US8, DC_REG_US3, DC_REG_US2,
  DC_REG_COUNT
};

/* Operation ids for dc_workspace_bytes. */
enum { DC_OP_DECODE = 0, DC_OP_MULTITENANT = 1, DC_OP_PREFILL = 2 };

/* Human-readable name of a status code (static string, never NULL). */
const char* dc_status_string(dc_status s);

/* Checks a spec against the shape rules (DC_OK or DC_ERR_SHAPE /
 * DC_ERR_INVALID_ARG for NULL). */
dc_status dc_check_spec(const dc_spec* spec);

/* Size in bytes of the packed buffer of `spec` (0 if the spec is invalid). */
size_t dc_packed_bytes(const dc_spec* spec);

/* Bytes the kept pairs need without padding: codes + 4 B of scale/zero per
 * 128-element group + 4 B of sigma per pair.  This is the "algorithmic"
 * packed-delta byte count used for bandwidth figures. */
size_t dc_algorithmic_bytes(const dc_spec* spec);

/* Byte offset and size of region `region` (DC_REG_*) inside the buffer. */
dc_status dc_region(const dc_spec* spec, int32_t region, size_t* offset, size_t* size);

/*
 * dc_pack -- quantize and pack one delta (host, synchronous, deterministic).
 * [P1] technical principles and [P2] "Approach": pairs ordered by descending
 * singular value, the first n8 at 8 bits, the next n3 at 3, the next n2 at 2.
 *   U      host fp32 [r][out], row i = u_i (r = n8+n3+n2 rows are read)
 *   sigma  host fp32 [r], stored unquantized
 *   V      host fp32 [r][in], row i = v_i
 *   out    host buffer of out_bytes >= dc_packed_bytes(spec); fully written
 * Quantizer, per 128-element group w of one vector at b bits, in fp64:
 *   mn = min(0, min w), mx = max(0, max w), maxq = 2^b-1,
 *   s_h = fp16_RNE((mx-mn)/maxq) (direct fp64 -> fp16; 1.0 if it is 0),
 *   z = clamp(rint(-mn/s_h), 0, maxq), q = clamp(rint(w/s_h) + z, 0, maxq),
 *   rint = round half to even.
 * Errors: DC_ERR_INVALID_ARG (NULL), DC_ERR_SHAPE, DC_ERR_BUFFER,
 * DC_ERR_RANGE (non-finite input, or s_h overflows fp16).  On error `out`
 * may be partly written.
 */
dc_status dc_pack(const dc_spec* spec, const float* U, const float* sigma, const float* V,
                  void* out, size_t out_bytes);

/*
 * dc_pack_device -- dc_pack on the GPU (asynchronous on `stream`).  The same
 * quantizer and format, bit for bit: onboarding a tenant's delta without a
 * round trip through host memory.  [P1] technical principles and [P2]
 * "Approach" as for dc_pack.
 *   U, sigma, V  device fp32, layouts of dc_pack (U and V 8-byte aligned)
 *   out          device buffer of out_bytes >= dc_packed_bytes(spec),
 *                16-byte aligned; fully written (padding zeroed)
 *   flag         device uint32, set to 0 by the call and to 1 if an input
 *                is non-finite or a scale overflows fp16 (then `out` is
 *                unspecified); read it after synchronizing the stream
 * Host checks, before anything is enqueued: DC_ERR_INVALID_ARG (NULL),
 * DC_ERR_SHAPE, DC_ERR_ALIGN, DC_ERR_BUFFER, DC_ERR_UNSUPPORTED (a packed
 * buffer of 2 GiB or more); DC_ERR_HIP if a launch fails.  Allocates
 * nothing; writes only `out` and `flag`.
 */
dc_status dc_pack_device(const dc_spec* spec, const float* U, const float* sigma, const float* V,
                         void* out, size_t out_bytes, uint32_t* flag, void* stream);

/*
 * dc_allocate_bits -- one bit width per singular pair for a storage budget
 * (host, synchronous, deterministic).  [P4] "Enhancing Delta Compression in
 * LLMs via SVD-based Quantization Error Minimization", §2.2: the widths
 * minimize the summed quantization error subject to a bit budget, one width
 * per row, widths from a candidate set (a 0/1 integer program; §2.1 eq. 5
 * gives the error of row i as about Sigma_ii^2 * Delta V_i X X^T Delta V_i^T
 * for calibration samples X).  Solved exactly as a multiple-choice knapsack
 * by dynamic programming over the budget used: time r * (budget+1) * nb,
 * memory r * (budget+1) bytes.
 *   r       pairs
 *   nb      candidate widths, 1..127
 *   cost    host int32 [nb], storage units of each candidate (>= 0); with
 *           this format a pair at b bits stores b * (out + in) bits, so
 *           cost = b and budget = the allowed sum of widths
 *   err     host double [r][nb], error of pair i at candidate k (finite)
 *   budget  total units allowed
 *   choice  host int32 [r], written: the candidate index of each pair
 *   total   host double, written if not NULL: the least total error
 * A row's candidates are tried in index order and a later one replaces an
 * earlier one only if strictly better; among end states of equal error the
 * one using the least budget wins.  Errors: DC_ERR_INVALID_ARG (NULL, r < 0,
 * nb out of range, a negative cost, a non-finite error), DC_ERR_RANGE (no
 * choice fits the budget), DC_ERR_UNSUPPORTED (r * (budget+1) of 2^31 or
 * more).  Allocates host memory for its tables; writes only choice, total.
 */
dc_status dc_allocate_bits(int32_t r, int32_t nb, const int32_t* cost, const double* err, int64_t budget,
                           int32_t* choice, double* total);

/*
 * dc_error_table -- the error table of dc_allocate_bits on the GPU
 * (asynchronous on `stream`).  [P4] "Enhancing Delta Compression in LLMs via
 * SVD-based Quantization Error Minimization", §2.1 eq. 5: quantizing row i of
 * V at b bits costs about sigma_i^2 ||(V̂_i - V_i) X||^2 for calibration
 * samples X; V̂_i is the row quantized by this library's quantizer (the one of
 * dc_pack: 128-element groups, fp16 scale and zero) and dequantized to its
 * fp16 values; width 0 drops the row (V̂_i = 0).
 *   r, in    rows of V and their length (in a positive multiple of 128)
 *   ncal     calibration samples (columns of X), >= 1
 *   sigma    device fp32 [r]
 *   V        device fp32 [r][in], row i = v_i, 8-byte aligned
 *   X        device fp32 [in][ncal] (one sample per column)
 *   widths   host int32 [nw], each 0..8; 1 <= nw <= DC_ERR_MAX_WIDTHS
 *   err      device fp64 [r][nw], written: err[i*nw + k] for widths[k]
 *   flag     device uint32, set to 0 by the call and to 1 if an input is
 *            non-finite or a scale overflows fp16
 *   ws       device workspace of ws_bytes >= dc_error_table_workspace_bytes
 * Arithmetic: the differences V̂_i - V_i in fp32 (exact), the products with X
 * in fp32, their squares and sums in fp64, in a fixed order.  Errors:
 * DC_ERR_INVALID_ARG (NULL, r < 0, ncal < 1, nw or a width out of range),
 * DC_ERR_SHAPE, DC_ERR_ALIGN, DC_ERR_BUFFER, DC_ERR_UNSUPPORTED (more than
 * 2^31 elements in V, X or the workspace's difference rows).
 */
#define DC_ERR_MAX_WIDTHS 8
size_t dc_error_table_workspace_bytes(int32_t r, int32_t in, int32_t nw);
dc_status dc_error_table(int32_t r, int32_t in, int32_t ncal, const float* sigma, const float* V, const float* X,
                         const int32_t* widths, int32_t nw, double* err, uint32_t* flag, void* ws,
                         size_t ws_bytes, void* stream);

/*
 * dc_svd -- the r leading singular pairs of a delta on the GPU: the first
 * step of compressing it ([P1] technical principles: the delta's low-rank
 * decomposition; [P4] §2.4 step 1: SVD of the delta, then bit allocation and
 * quantization), so that a tenant can be onboarded without a host SVD.  The
 * outputs are dc_pack_device's inputs.  Synchronous: returns when they are
 * written (it waits on `stream` between sweeps).
 *   delta   device fp32 [out][in] row-major, 4-byte aligned; out, in >= 1
 *   r       pairs wanted, 0 <= r <= min(out, in)
 *   U       device fp32 [r][out], row i = u_i
 *   sigma   device fp32 [r], descending (index order on ties)
 *   V       device fp32 [r][in], row i = v_i
 *   ws      device workspace, 256-byte aligned, of ws_bytes >=
 *           dc_svd_workspace_bytes(out, in) (about 16 m^2 bytes for
 *           m = min(out, in))
 *   sweeps  host int32 or NULL: Jacobi sweeps run
 * Each pair is signed so that the largest-magnitude entry of v_i is positive
 * (lowest index on ties); for sigma_i = 0 the vector derived from the other
 * (u_i when out >= in, else v_i) is zero.
 * Method: G = A^T A (in <= out) or A A^T, m x m, summed in fp64 from the
 * fp32 entries; its eigenpairs by block Jacobi (32-index blocks, pairs of
 * blocks diagonalized in LDS, sweeps of a round-robin tournament) until every
 * pair of a sweep is diagonal to |G_ab| <= 1e-13 (sqrt(|G_aa G_bb|) +
 * trace(G) / 10); sigma_i = sqrt(lambda_i) and the other vectors as
 * A v_i / sigma_i (resp. A^T u_i / sigma_i) in fp64 sums.  Accuracy:
 * sigma_i to about 1e-16 sigma_1^2 / sigma_i^2 relative (the Gram matrix
 * squares the condition), vectors to about 1e-14 trace(G) over the gap
 * between their eigenvalue and the neighbouring ones.
 * Errors: DC_ERR_INVALID_ARG (NULL, r out of range), DC_ERR_SHAPE (out or
 * in < 1), DC_ERR_ALIGN, DC_ERR_BUFFER, DC_ERR_UNSUPPORTED (min(out, in) >
 * 16384, or out * in of 2^31 or more), DC_ERR_RANGE (a non-finite entry, or
 * no convergence within 40 sweeps: outputs unspecified), DC_ERR_HIP.
 * Allocates nothing; writes U, sigma, V and the workspace.
 */
size_t dc_svd_workspace_bytes(int32_t out, int32_t in);
dc_status dc_svd(int32_t out, int32_t in, int32_t r, const float* delta, float* U, float* sigma, float* V, void* ws,
                 size_t ws_bytes, int32_t* sweeps, void* stream);

/*
 * dc_pack_codes -- pack already-quantized codes (host, synchronous).
 *   codes_u  host uint8 [r][out], code of u_i at row o (< 2^b of its segment)
 *   codes_v  host uint8 [r][in]
 *   sz_u     host uint16 [r][out/128][2]: (fp16 scale bits, fp16 zero bits)
 *   sz_v     host uint16 [r][in/128][2]
 *   sigma    host fp32 [r]
 * Errors: DC_ERR_INVALID_ARG (NULL), DC_ERR_SHAPE, DC_ERR_BUFFER,
 * DC_ERR_RANGE (a code does not fit its segment's width).
 */
dc_status dc_pack_codes(const dc_spec* spec, const uint8_t* codes_u, const uint8_t* codes_v,
                        const uint16_t* sz_u, const uint16_t* sz_v, const float* sigma,
                        void* out, size_t out_bytes);

/*
 * dc_unpack -- inverse of dc_pack_codes (host, synchronous).  Reads
 * dc_packed_bytes(spec) bytes of `packed` (host); writes the five arrays in
 * the layouts of dc_pack_codes.  Errors: DC_ERR_INVALID_ARG, DC_ERR_SHAPE,
 * DC_ERR_BUFFER (packed_bytes too small).
 */
dc_status dc_unpack(const dc_spec* spec, const void* packed, size_t packed_bytes,
                    uint8_t* codes_u, uint8_t* codes_v, uint16_t* sz_u, uint16_t* sz_v,
                    float* sigma);

/*
 * dc_workspace_bytes -- device workspace that one call of `op` needs.
 *   specs  host array of n specs (the tenants' specs; n = 1 for decode)
 *   T      tokens of the call
 * Returns 0 on invalid arguments.
 */
size_t dc_workspace_bytes(int32_t op, const dc_spec* specs, int32_t n, int32_t T);

/*
 * dc_apply_decode -- one tenant, T tokens.  [P2] "Key results" (the GPU
 * kernel that applies the mixed-precision delta); [P1] technical principles.
 *   d       host struct; d->base is device memory holding the packed delta
 *   W_base  device bf16 [out][in] (nn.Linear layout), or NULL = delta only
 *   x       device bf16 [T][in]
 *   y       device bf16 [T][out], fully overwritten with
 *           RNE_bf16(W_base x + U diag(sigma) V x), sums in fp32, rounded once
 *   ws      device workspace of ws_bytes >= dc_workspace_bytes(DC_OP_DECODE,..)
 *   stream  hipStream_t
 * T = 0 is a no-op returning DC_OK.  x and y must not overlap.
 * Summation order is fixed, so repeated calls give the same bits: V x is
 * summed over slices of 2048 inputs and, for T <= 256, W_base x over K
 * ranges of 512; two partials are added onto zero (order-independent), more
 * are added in slice (range) order by the work item that finishes last.
 * Batches of more than 256 tokens compute W_base x in tiles of 128 x 128
 * (another fixed order, so they may round differently from smaller batches).
 */
dc_status dc_apply_decode(const dc_delta_view* d, const uint16_t* W_base, const uint16_t* x,
                          uint16_t* y, int32_t T, void* ws, size_t ws_bytes, void* stream);

/*
 * dc_apply_multitenant -- n tenants over one backbone, tokens routed by id.
 * [P1] application scenarios (multi-tenant serving); [P2] "Key results" (50
 * models on one GPU).
 *   views       host array [n] (n <= DC_MAX_TENANTS); all with the same
 *               out/in; n8/n3/n2 may differ per tenant
 *   W_base      device bf16 [out][in] or NULL
 *   x           device bf16 [T][in]
 *   tenant_ids  device int32 [T]; id k in [0,n) selects views[k]; -1 means
 *               backbone only.  Any other id is a contract violation: the
 *               token is served backbone-only and bit 0 of the uint32 at byte
 *               0 of ws is set (the word is cleared by every call).
 *   y           device bf16 [T][out], fully overwritten, original token order
 * Routing happens on the device; the call never reads the ids on the host.
 */
dc_status dc_apply_multitenant(const dc_delta_view* views, int32_t n, const uint16_t* W_base,
                               const uint16_t* x, const int32_t* tenant_ids, uint16_t* y,
                               int32_t T, void* ws, size_t ws_bytes, void* stream);

/*
 * dc_apply_multitenant_group -- m matrices that read the same input with
 * the same tenant routing (q, k and v of attention; gate and up of the MLP)
 * in one call: the tokens are routed and x is staged once, and each kernel
 * covers all m matrices in one launch.  [P1] application scenarios
 * (multi-tenant serving); [P2] "Key results" (50 models on one GPU).
 *   views       host array [m][n]: views[j*n + k] is tenant k's delta of
 *               matrix j; every matrix has the same in; within a matrix
 *               every tenant has the same out (out may differ between
 *               matrices, e.g. grouped-query k and v)
 *   m           1 .. DC_MAX_GROUP
 *   W_base      host array [m] of device bf16 [out_j][in] pointers, or NULL
 *               (every matrix delta only); a NULL entry makes that matrix
 *               delta only
 *   x, tenant_ids, T   as dc_apply_multitenant
 *   y           host array [m] of device bf16 [T][out_j], fully overwritten
 *   ws          ws_bytes >= dc_group_workspace_bytes(specs of views, m, n, T)
 * Output j is bit-identical to dc_apply_multitenant on matrix j alone.
 * Errors as dc_apply_multitenant; DC_ERR_SHAPE if the matrices' in differ,
 * DC_ERR_UNSUPPORTED if m > DC_MAX_GROUP, DC_ERR_INVALID_ARG if outputs
 * overlap each other or x.  The status word of invalid ids is at byte 0 of
 * ws as for dc_apply_multitenant.
 */
dc_status dc_apply_multitenant_group(const dc_delta_view* views, int32_t m, int32_t n,
                                     const uint16_t* const* W_base, const uint16_t* x,
                                     const int32_t* tenant_ids, uint16_t* const* y, int32_t T,
                                     void* ws, size_t ws_bytes, void* stream);

/* Workspace of dc_apply_multitenant_group: specs [m][n] as its views; 0 on
 * invalid arguments. */
size_t dc_group_workspace_bytes(const dc_spec* specs, int32_t m, int32_t n, int32_t T);

/*
 * dc_apply_multitenant_timed -- dc_apply_multitenant that also records
 * caller-owned HIP events on `stream` between its kernels, so a caller can
 * time each stage (hipEventElapsedTime) without a profiler.
 *   events  host array of DC_STAGE_COUNT + 1 hipEvent_t (as void*); entry s
 *           is recorded just before stage s is enqueued, the last entry
 *           after the final stage; NULL entries are skipped.  A stage that
 *           does not run (no backbone, no ranks) leaves its start and the
 *           next stage's start on the same point of the stream.
 * Results are identical to dc_apply_multitenant.
 */
enum { DC_STAGE_ROUTE = 0, DC_STAGE_XPREP, DC_STAGE_BASE, DC_STAGE_VSIDE, DC_STAGE_USIDE,
       DC_STAGE_COUNT };
/* dc_apply_multitenant_group with the same stage events (each stage covers
 * the whole group). */
dc_status dc_apply_multitenant_group_timed(const dc_delta_view* views, int32_t m, int32_t n,
                                           const uint16_t* const* W_base, const uint16_t* x,
                                           const int32_t* tenant_ids, uint16_t* const* y, int32_t T,
                                           void* ws, size_t ws_bytes, void* stream, void* const* events);
dc_status dc_apply_multitenant_timed(const dc_delta_view* views, int32_t n, const uint16_t* W_base,
                                     const uint16_t* x, const int32_t* tenant_ids, uint16_t* y,
                                     int32_t T, void* ws, size_t ws_bytes, void* stream,
                                     void* const* events);

/*
 * dc_apply_multitenant_noalloc -- dc_apply_multitenant for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments without the
 * workspace: the call uses the library's own scratch array of
 * DC_SCRATCH_BYTES on the current device, a file-scope device array that
 * every GPU the library runs on holds until the process ends.  The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine);
 * its first call on a device looks the array's address up once.
 *   Limit: a call whose workspace (dc_workspace_bytes(DC_OP_MULTITENANT,..))
 *   exceeds DC_SCRATCH_BYTES returns DC_ERR_UNSUPPORTED and enqueues nothing.
 *   Sharing: every call on one GPU uses the same array, which keeps the last
 *   call's contents (each call writes what it reads before reading it).
 *   Calls on one GPU that overlap in time (different streams, or host
 *   threads without ordering) race on the array: the caller must order them.
 *   The status word of invalid ids lives in the array and is not returned;
 *   such tokens are still served backbone-only.
 * Results are identical to dc_apply_multitenant with a workspace of its own.
 */
#define DC_SCRATCH_BYTES (32u << 20)
dc_status dc_apply_multitenant_noalloc(const dc_delta_view* views, int32_t n, const uint16_t* W_base,
                                       const uint16_t* x, const int32_t* tenant_ids, uint16_t* y,
                                       int32_t T, void* stream);

/*
 * dc_apply_prefill -- n tenants, tokens grouped by tenant: tokens
 * seg_offsets[k] .. seg_offsets[k+1]-1 belong to views[k].  The prompt
 * phase of serving many fine-tuned models over one backbone: [P1]
 * application scenarios (multi-tenant serving of many fine-tuned models);
 * [P2] "Key results" (50 models served from one GPU) and "Experimental
 * setup" (13B backbones).
 *   seg_offsets  host int32 [n+1], non-decreasing, seg_offsets[0] = 0;
 *                T = seg_offsets[n]
 *   x, y         device bf16 [T][in], [T][out]
 * Same conventions as dc_apply_multitenant (the status word at byte 0 of ws
 * is cleared).  When every non-empty segment has at least 256 tokens and the
 * workspace holds the dense form's buffers, the call takes a dense form: per
 * tenant, t = sigma (V x) and y = W x + U t run as tiled matrix-core products
 * over the segment whose V and U operand tiles are dequantized from the
 * packed codes in registers (the fp16 values fp16(s (q - z)), exactly), x
 * entering as fp16 after a power-of-two rescale per token (exact for bf16
 * values within 2^24 of the token's largest) and t as fp16 hi + lo after a
 * power-of-two rescale per token (about 22 significant bits); fp32 sums in a
 * fixed order, so repeated calls give the same bits.  The products of up to 8
 * tenants run in one launch.  Otherwise the call takes the decode kernels of
 * dc_apply_multitenant.  The workspace for DC_OP_PREFILL (dc_workspace_bytes)
 * includes the dense form's buffers when T >= 256: fp32 t [T][rp] and 8 bytes
 * per token, rp = max over tenants of pad32(n8) + pad32(n3) + pad32(n2)
 * rounded up to 128 (at least 128).  A workspace of the DC_OP_MULTITENANT
 * size is also accepted (no dense form).
 * Weights: the dense form multiplies by the fp16 dequantized values
 * fp16(s (q - z)); the decode kernels multiply 8-bit pairs by the same fp16
 * values but 3- and 2-bit pairs by the exact grid values s (q - z), within
 * half an fp16 unit of them (the zero point is folded out of their sums).
 */
dc_status dc_apply_prefill(const dc_delta_view* views, int32_t n, const uint16_t* W_base,
                           const uint16_t* x, const int32_t* seg_offsets, uint16_t* y,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * dc_dequant -- the dequantized fp16 singular vectors, for tests.
 *   u_fp16  device fp16 bits [r][out], row i = fp16(s*(q-z)) of u_i
 *   v_fp16  device fp16 bits [r][in]
 * Values are bit-identical to the quantizer's definition above.
 */
dc_status dc_dequant(const dc_delta_view* d, uint16_t* u_fp16, uint16_t* v_fp16, void* stream);

/*
 * Baselines.  The pages compare Delta-CoMe, at the same storage, with a
 * low-rank delta and with BitDelta's 1-bit delta: [P2] "Experimental setup"
 * (baselines: low-rank SVD compression and BitDelta) and "Key results"
 * (Delta-CoMe ahead of both at 1/16); [P2] "Approach" (Delta-CoMe the size
 * of BitDelta); [P3] "Delta-CoMe: 大型语言模型的无需训练的混合精度增量压缩"
 * (related work: BitDelta quantizes a fine-tuning delta to 1 bit).  Neither
 * baseline's arithmetic is printed there; this library serves them as:
 *   DC_KIND_LOWRANK   the top r singular pairs as fp16 vectors, fp32 sigma:
 *                     y = W_base x + U (sigma * (V x)); at the budget of
 *                     Delta-CoMe's 1/16, r = floor(out in / (16 (out + in)))
 *                     (128 for 4096 x 4096)
 *   DC_KIND_BITDELTA  one sign bit per delta entry and one fp32 scale alpha:
 *                     y = W_base x + alpha S x, S in {+1, -1}^(out x in)
 * Formats (each region at a multiple of 256 bytes from the buffer start;
 * total rounded up to 256 bytes; pad entries zero):
 *   low-rank   SIGMA fp32 [r]; V fp16 [ceil(r/16)][in/32][64][8]: v_i[k] at
 *              tile i/16, step k/32, slot (i%16) + 16((k%32)/8), element
 *              k%8; U fp16 [out/16][ceil(r/32)][64][8]: u_i[o] at tile o/16,
 *              step i/32, slot (o%16) + 16((i%32)/8), element i%8.  One
 *              16-row tile of one 32-element step is 1 KiB, a matrix-core
 *              operand for 64 lanes.
 *   BitDelta   SCALE fp32 alpha (region of 256 bytes), then uint32 words
 *              [out/16][in/128][4][16]: word (T, g, c, i) holds the signs of
 *              row 16T+i, columns 128g + 32c + k (k < 32), bit set = +1; entry
 *              k sits at bit 4(k'%8) + k'/8 with k' = k/2 for even k and
 *              16 + k/2 for odd k, so that word >> s & 0x11111111 (s < 4) holds
 *              8 entries, one per nibble.
 * Shapes: out and in positive multiples of 128; low-rank 0 <= r <= min(out,
 * in).  Calls and conventions as for the Delta-CoMe calls.
 */
enum { DC_KIND_LOWRANK = 1, DC_KIND_BITDELTA = 2 };

typedef struct dc_baseline_view {
  int32_t kind;     /* DC_KIND_LOWRANK or DC_KIND_BITDELTA */
  int32_t out, in;  /* matrix shape, multiples of 128 */
  int32_t r;        /* low-rank: pairs kept; BitDelta: 0 */
  const void* base; /* device pointer to dc_baseline_bytes(kind, out, in, r) bytes */
} dc_baseline_view;

/* Size in bytes of a baseline buffer; 0 if the arguments are invalid (and
 * for a low-rank delta with r = 0, which stores nothing and may have a NULL
 * base). */
size_t dc_baseline_bytes(int32_t kind, int32_t out, int32_t in, int32_t r);

/* Bytes the baseline must move without padding (bandwidth figures):
 * low-rank 2 r (out + in) + 4 r; BitDelta out in / 8 + 4. */
size_t dc_baseline_algorithmic_bytes(int32_t kind, int32_t out, int32_t in, int32_t r);

/*
 * dc_pack_lowrank -- lay out fp16 pairs in the low-rank format (host).
 *   U      host fp16 bits [r][out], row i = u_i
 *   sigma  host fp32 [r]
 *   V      host fp16 bits [r][in], row i = v_i
 *   dst    host buffer of dst_bytes >= dc_baseline_bytes(DC_KIND_LOWRANK, ..),
 *          fully written
 * Errors: DC_ERR_INVALID_ARG (NULL with r > 0), DC_ERR_SHAPE, DC_ERR_BUFFER.
 */
dc_status dc_pack_lowrank(int32_t out, int32_t in, int32_t r, const uint16_t* U, const float* sigma,
                          const uint16_t* V, void* dst, size_t dst_bytes);

/*
 * dc_pack_bitdelta -- lay out sign bits and their scale in the BitDelta
 * format (host).
 *   signs  host uint8 [out][in], nonzero = +1, 0 = -1
 *   alpha  the scale (finite)
 *   dst    host buffer of dst_bytes >= dc_baseline_bytes(DC_KIND_BITDELTA, ..)
 * Errors: DC_ERR_INVALID_ARG (NULL), DC_ERR_SHAPE, DC_ERR_BUFFER,
 * DC_ERR_RANGE (alpha not finite).
 */
dc_status dc_pack_bitdelta(int32_t out, int32_t in, const uint8_t* signs, float alpha, void* dst,
                           size_t dst_bytes);

/* Workspace of dc_apply_baseline_multitenant(_group): views [m][n] as its
 * views; 0 on invalid arguments. */
size_t dc_baseline_workspace_bytes(const dc_baseline_view* views, int32_t m, int32_t n, int32_t T);

/*
 * dc_apply_baseline_multitenant -- dc_apply_multitenant for baseline
 * deltas: n tenants of one kind over one backbone, tokens routed by id
 * (-1 = backbone only; other ids out of range as for dc_apply_multitenant).
 *   views  host array [n], one kind, one out/in (low-rank r may differ)
 *   W_base, x, tenant_ids, y, T, ws, ws_bytes, stream  as dc_apply_multitenant
 * y = RNE_bf16(W_base x + delta x), fp32 sums in a fixed order (repeated
 * calls give the same bits).  Arithmetic: BitDelta multiplies x as two fp8
 * (e4m3) pieces with power-of-two block scales (about 2^-8 relative per
 * element) by the exact signs; low-rank multiplies x, rescaled by a power of
 * two per 128 inputs into fp16 (exact for bf16 values in fp16's normal
 * range), by the fp16 V, and sigma (V x), split into two fp16 pieces per
 * token, by the fp16 U.
 * Errors: as dc_apply_multitenant; DC_ERR_SHAPE for mixed kinds or shapes.
 */
dc_status dc_apply_baseline_multitenant(const dc_baseline_view* views, int32_t n, const uint16_t* W_base,
                                        const uint16_t* x, const int32_t* tenant_ids, uint16_t* y, int32_t T,
                                        void* ws, size_t ws_bytes, void* stream);

/* The grouped form (as dc_apply_multitenant_group): views [m][n], one kind
 * for the whole group, W_base and y host arrays [m]; output j is
 * bit-identical to dc_apply_baseline_multitenant on matrix j alone. */
dc_status dc_apply_baseline_multitenant_group(const dc_baseline_view* views, int32_t m, int32_t n,
                                              const uint16_t* const* W_base, const uint16_t* x,
                                              const int32_t* tenant_ids, uint16_t* const* y, int32_t T,
                                              void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DELTACOME_H */
