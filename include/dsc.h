/*
 * dsc.h -- C ABI of the MI355X (gfx950) causal dynamic short convolution library.
 *
 * The operation ("Dynamic Short Convolutions Improve Transformers", technical
 * summary page, section Metodologia, bullet Mecanismo) is, for every sequence
 * b, step t and channel c:
 *
 *     y[b,t,c] = residual * x[b,t,c] + sum_{k=0}^{W-1} f[b,t,c,k] * x[b,t-k,c]
 *
 * with x[b,t<0,c] = 0 (each sequence starts from zero history). The filter f
 * is input-dependent, drawn fresh at every step, in one of two forms (same
 * section, bullet Parametrizacao):
 *   - head-wise tying: f[b,t,c,k] = w[b,t,c/Hc,k], one filter per head of
 *     Hc = D/G consecutive channels;
 *   - low-rank: f[b,t,c,k] = sum_r z[b,t,r] * U[r, c*W+k], generated on-chip
 *     and never written to memory (section "Kernel de Fatoracao de Baixo Posto
 *     Fundido").
 * The residual flag gives the X + dynamicShortConv(X) form of bullet
 * Posicionamento. The backward entry points return the gradients of that
 * forward pass (the chain rule; the page trains with it but prints no
 * backward formulas).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors: device pointers to contiguous row-major arrays:
 *     x, y, dy, dx   [B, T, D]
 *     w, dw          [B, T, G, W]        (head-wise)
 *     z, dz          [B, T, R]           (low-rank)
 *     U, dU          [R, D*W]            (column c*W+k is channel c, tap k)
 *   All tensors of one call share one dtype. Arithmetic is float32 in
 *   registers; bfloat16 outputs are rounded to nearest-even.
 * Ownership: the caller allocates and frees everything, including the
 *   low-rank backward's workspace. The library never allocates, frees,
 *   synchronises or keeps a pointer after returning. (The one exception is
 *   dsc_lowrank_bwd_noalloc, whose fixed-size scratch array is part of the
 *   library's device image.) Work is enqueued on
 *   `stream` (a hipStream_t; NULL is the default stream) and the caller keeps
 *   every buffer alive until that work has completed.
 * Outputs are overwritten, never accumulated into. No output may overlap an
 *   input or another output (DSC_ERROR_ALIASING): in particular y = x in place
 *   is refused, because later steps still read the old x.
 * Errors are checked before anything is enqueued, in this order:
 *   B < 0 or T < 0                                   -> DSC_ERROR_INVALID_VALUE
 *   B == 0 or T == 0                                 -> DSC_SUCCESS, nothing done
 *   D <= 0, G <= 0, D % G != 0, W outside [1, 8],
 *   R outside [1, 128], unknown dtype, null pointer  -> DSC_ERROR_INVALID_VALUE
 *   a pointer not 16-byte aligned, or D not a
 *   multiple of 8 (bf16) or of 4 (fp32)               -> DSC_ERROR_MISALIGNED
 *   overlapping output                                -> DSC_ERROR_ALIASING
 *   workspace smaller than the query returns          -> DSC_ERROR_WORKSPACE
 *   a failed kernel launch                            -> DSC_ERROR_HIP
 *   Faults inside a kernel surface at the caller's next synchronisation.
 * Nothing is printed and no C++ exception crosses this interface. Calls are
 *   re-entrant and keep no global state beyond a per-device address cache;
 *   calls that share a workspace race.
 */
#ifndef DSC_H_
#define DSC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSC_ABI_VERSION 8

typedef enum { DSC_F32 = 0, DSC_BF16 = 1 } dsc_dtype_t;

typedef enum {
  DSC_SUCCESS = 0,
  DSC_ERROR_INVALID_VALUE = 1,
  DSC_ERROR_MISALIGNED = 2,
  DSC_ERROR_ALIASING = 3,
  DSC_ERROR_NOT_SUPPORTED = 4,
  DSC_ERROR_WORKSPACE = 5,
  DSC_ERROR_HIP = 6
} dsc_status_t;

typedef void* dsc_stream_t; /* a hipStream_t */

/* Head-wise forward (Mecanismo + head-wise tying + Posicionamento):
 *   y[b,t,c] = residual*x[b,t,c] + sum_k w[b,t,c/Hc,k] * x[b,t-k,c],  Hc = D/G.
 * x [B,T,D] in, w [B,T,G,W] in, y [B,T,D] out. residual is 0 or 1. */
dsc_status_t dsc_fwd(const void* x, const void* w, void* y, int64_t B, int64_t T, int64_t D,
                     int64_t G, int32_t W, int32_t residual, dsc_dtype_t dtype,
                     dsc_stream_t stream);

/* Head-wise backward: given dy = dL/dy, writes
 *   dx[b,s,c]   = residual*dy[b,s,c] + sum_k w[b,s+k,c/Hc,k] * dy[b,s+k,c]   (s+k < T)
 *   dw[b,t,h,k] = sum_{c in head h} dy[b,t,c] * x[b,t-k,c]                   (0 if t < k)
 * x, dy [B,T,D] and w [B,T,G,W] in; dx [B,T,D] and dw [B,T,G,W] out, both in one pass. */
dsc_status_t dsc_bwd(const void* x, const void* w, const void* dy, void* dx, void* dw, int64_t B,
                     int64_t T, int64_t D, int64_t G, int32_t W, int32_t residual,
                     dsc_dtype_t dtype, dsc_stream_t stream);

/* Low-rank forward (low-rank factorisation; fused-kernel section):
 *   f[b,t,c,k] = sum_r z[b,t,r] * U[r,c*W+k]   (registers only, never stored)
 *   y[b,t,c]   = residual*x[b,t,c] + sum_k f[b,t,c,k] * x[b,t-k,c]
 * x [B,T,D], z [B,T,R], U [R,D*W] in; y [B,T,D] out. */
dsc_status_t dsc_lowrank_fwd(const void* x, const void* z, const void* U, void* y, int64_t B,
                             int64_t T, int64_t D, int32_t R, int32_t W, int32_t residual,
                             dsc_dtype_t dtype, dsc_stream_t stream);

/* Bytes of device workspace dsc_lowrank_bwd needs for these sizes (0 when
 * B*T == 0 or the arguments are invalid). The workspace holds float32
 * partial sums of dz and dU; its contents on entry do not matter. */
size_t dsc_lowrank_bwd_workspace_bytes(int64_t B, int64_t T, int64_t D, int32_t R, int32_t W,
                                       dsc_dtype_t dtype);

/* Low-rank backward: given dy, with g[b,t,c,k] = dy[b,t,c] * x[b,t-k,c] (0 if t < k), writes
 *   dx[b,s,c] = residual*dy[b,s,c] + sum_k f[b,s+k,c,k] * dy[b,s+k,c]   (s+k < T)
 *   dz[b,t,r] = sum_{c,k} g[b,t,c,k] * U[r,c*W+k]
 *   dU[r,c*W+k] = sum_{b,t} z[b,t,r] * g[b,t,c,k]
 * x, dy [B,T,D], z [B,T,R], U [R,D*W] in; dx [B,T,D], dz [B,T,R], dU [R,D*W] out.
 * workspace: device memory of at least dsc_lowrank_bwd_workspace_bytes(...) bytes,
 * 16-byte aligned, owned by the caller (may be NULL when that query returns 0).
 * Sums run in a fixed order: repeated calls give bit-identical results. */
dsc_status_t dsc_lowrank_bwd(const void* x, const void* z, const void* U, const void* dy, void* dx,
                             void* dz, void* dU, void* workspace, size_t workspace_bytes,
                             int64_t B, int64_t T, int64_t D, int32_t R, int32_t W,
                             int32_t residual, dsc_dtype_t dtype, dsc_stream_t stream);

/* Low-rank backward that allocates nothing, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving or training loops,
 * harnesses that forbid allocation). Same operation, arguments, checks and
 * kernels as dsc_lowrank_bwd, without the workspace: the float32 partial sums go
 * to a scratch array of DSC_NOALLOC_SCRATCH_BYTES that the library holds on each
 * GPU it runs on (a static device array, present until the process ends).
 * Problems whose dsc_lowrank_bwd_workspace_bytes exceeds that size return
 * DSC_ERROR_WORKSPACE before anything is enqueued. The call uses no hipMalloc,
 * hipFree or allocating library routine; the first call on a device looks up the
 * array's address there (call it with the stream's device current). Every call on
 * one GPU shares that GPU's array and leaves its contents behind (nothing in it
 * needs clearing), so calls that may overlap on one GPU (other streams, other
 * threads) race and must be serialised by the caller. */
#define DSC_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
dsc_status_t dsc_lowrank_bwd_noalloc(const void* x, const void* z, const void* U, const void* dy,
                                     void* dx, void* dz, void* dU, int64_t B, int64_t T, int64_t D,
                                     int32_t R, int32_t W, int32_t residual, dsc_dtype_t dtype,
                                     dsc_stream_t stream);

/* ------------------------------------------------------- packed sequences
 *
 * Several sequences may share one row of the [B, T] layout (packed training
 * batches, or the short convolutions of recurrent hosts over concatenated
 * documents). pos [B, T] int32 (device) gives each token's index within its own
 * sequence: 0 at every sequence start, then 1, 2, ... Tap k > 0 of step t is
 * applied only if k <= pos[b,t] (and t-k >= 0), so no sequence sees another's
 * inputs; the forward definition (Mecanismo) is applied per sequence. The
 * gradients are those of that masked forward:
 *   dx[b,s,c]   sums the terms of steps s+k whose tap k exists,
 *   dw[b,t,h,k], dz and dU take g[b,t,c,k] = dy[b,t,c] * x[b,t-k,c] only where tap
 *                k of step t exists (0 elsewhere).
 * Positions are read on the device and never checked by the host; any values
 * define the masked operation above (pos >= W-1 everywhere is the dense one).
 * The page does not treat packing; this is its definition applied per sequence.
 * Arguments and checks are those of the dense calls, plus pos: non-null, 4-byte
 * aligned, overlapping no output. The low-rank backward's workspace is the size
 * dsc_lowrank_bwd_workspace_bytes returns for the same sizes. */

dsc_status_t dsc_fwd_varlen(const void* x, const void* w, const int32_t* pos, void* y, int64_t B, int64_t T,
                            int64_t D, int64_t G, int32_t W, int32_t residual, dsc_dtype_t dtype,
                            dsc_stream_t stream);

dsc_status_t dsc_bwd_varlen(const void* x, const void* w, const int32_t* pos, const void* dy, void* dx,
                            void* dw, int64_t B, int64_t T, int64_t D, int64_t G, int32_t W,
                            int32_t residual, dsc_dtype_t dtype, dsc_stream_t stream);

dsc_status_t dsc_lowrank_fwd_varlen(const void* x, const void* z, const void* U, const int32_t* pos, void* y,
                                    int64_t B, int64_t T, int64_t D, int32_t R, int32_t W, int32_t residual,
                                    dsc_dtype_t dtype, dsc_stream_t stream);

dsc_status_t dsc_lowrank_bwd_varlen(const void* x, const void* z, const void* U, const int32_t* pos,
                                    const void* dy, void* dx, void* dz, void* dU, void* workspace,
                                    size_t workspace_bytes, int64_t B, int64_t T, int64_t D, int32_t R,
                                    int32_t W, int32_t residual, dsc_dtype_t dtype, dsc_stream_t stream);

/* ------------------------------------------------- rotary embedding epilogue
 *
 * In the QKV placement the convolution runs on the Q, K and V projections
 * before the rotary position embedding (Posicionamento). These calls fuse the
 * two: the forward writes the convolution's output with its first d_rot
 * channels (the Q and K heads, head_dim channels each) already rotated, and the
 * backward rotates dy back (the transposed rotation) as it reads it, so Q and K
 * cross HBM once instead of three times. The rotation is RoFormer's: in each
 * head, pair i (i < head_dim/2) is the channels (i, i + head_dim/2), or
 * (2i, 2i+1) when interleaved, and (a, b) becomes
 *     (a*cos[p][i] - b*sin[p][i],  a*sin[p][i] + b*cos[p][i])
 * for the token's position p: pos[b,t] when pos is given (packed sequences,
 * with the convolution masked as in the *_varlen calls), else t. The tables are
 * the caller's (device, float32, [n_pos][head_dim/2], 16-byte aligned); p is
 * clamped to [0, n_pos-1], and without pos T must not exceed n_pos.
 * Requirements: head_dim a power of two in [16, 512], d_rot a multiple of
 * head_dim and at most D, interleaved 0 or 1 (DSC_ERROR_INVALID_VALUE
 * otherwise); channels per filter D/G a power of two up to 512
 * (DSC_ERROR_NOT_SUPPORTED otherwise). The tables and pos count as inputs for
 * the aliasing check. rope may not be NULL. */
typedef struct {
  const float* cos;      /* [n_pos][head_dim/2] */
  const float* sin;      /* [n_pos][head_dim/2] */
  int64_t n_pos;         /* rows of the tables */
  int64_t d_rot;         /* channels [0, d_rot) are rotated */
  int32_t head_dim;      /* channels per rotary head */
  int32_t interleaved;   /* 0: pairs (i, i + head_dim/2); 1: pairs (2i, 2i+1) */
} dsc_rope_t;

/* y = rotary(residual*x + head-wise convolution of x with w) on channels [0, d_rot).
 * x [B,T,D], w [B,T,G,W], pos [B,T] or NULL in; y [B,T,D] out. */
dsc_status_t dsc_fwd_rope(const void* x, const void* w, const int32_t* pos, const dsc_rope_t* rope, void* y,
                          int64_t B, int64_t T, int64_t D, int64_t G, int32_t W, int32_t residual,
                          dsc_dtype_t dtype, dsc_stream_t stream);

/* Gradients dx, dw of dsc_fwd_rope given dy = dL/dy: dsc_bwd (or dsc_bwd_varlen)
 * applied to the transposed rotation of dy. */
dsc_status_t dsc_bwd_rope(const void* x, const void* w, const int32_t* pos, const dsc_rope_t* rope,
                          const void* dy, void* dx, void* dw, int64_t B, int64_t T, int64_t D, int64_t G,
                          int32_t W, int32_t residual, dsc_dtype_t dtype, dsc_stream_t stream);

/* --------------------------------------------------- generator in the kernel
 *
 * The head-wise filter of step t is a learned linear map of the hidden state
 * (Parametrizacao): w[b,t,g,k] = sum_j h[b,t,j] * Wg[g*W+k, j], Wg stored like a
 * linear layer's weight, [G*W, K]. dsc_fwd_gen computes that product on the
 * matrix cores and convolves with it in the same kernel,
 *     y[b,t,c] = residual*x[b,t,c] + sum_k w[b,t,c/Hc,k] * x[b,t-k,c],
 * so w never reaches HBM; w is kept in float32 (not rounded to bf16).
 * x [B,T,D], h [B,T,K], Wg [G*W,K] in; y [B,T,D] out. bf16 only.
 * Requirements beyond the shared conventions (DSC_ERROR_NOT_SUPPORTED otherwise):
 * G a multiple of 32, D/G a multiple of 8, K a multiple of 64, and the per-row
 * ranges T*K, G*W*K, T*D below 2^30 elements. The gradients: dsc_bwd_gen below
 * gives dx and dw; dh = dw . Wg and dWg = dw^T . h are then plain GEMMs. */
dsc_status_t dsc_fwd_gen(const void* x, const void* h, const void* Wg, void* y, int64_t B, int64_t T,
                         int64_t D, int64_t G, int32_t W, int64_t K, int32_t residual, dsc_dtype_t dtype,
                         dsc_stream_t stream);

/* dsc_fwd_gen on packed sequences: pos [B,T] (int32, device) as for dsc_fwd_varlen,
 * tap k of step t applied only if k <= pos[b,t]. */
dsc_status_t dsc_fwd_gen_varlen(const void* x, const void* h, const void* Wg, const int32_t* pos, void* y,
                                int64_t B, int64_t T, int64_t D, int64_t G, int32_t W, int64_t K,
                                int32_t residual, dsc_dtype_t dtype, dsc_stream_t stream);

/* Gradients of dsc_fwd_gen given dy = dL/dy (the chain rule through the
 * forward above; Parametrizacao trains the generator with the rest of the model):
 *     dx[b,s,c]   = residual*dy[b,s,c] + sum_k w[b,s+k,c/Hc,k] * dy[b,s+k,c]  (s+k < T)
 *     dw[b,t,g,k] = sum_{c in head g} dy[b,t,c] * x[b,t-k,c]                   (t-k >= 0)
 * with w regenerated from h and Wg on the matrix cores exactly as in the forward
 * (float32, never written to HBM). x, dy [B,T,D], h [B,T,K], Wg [G*W,K] in;
 * dx [B,T,D] and dw [B,T,G,W] (bf16, the layout of dsc_bwd's dw) out, overwritten.
 * dw is what the generator's own gradients need: dh = dw . Wg, dWg = dw^T . h.
 * Requirements: those of dsc_fwd_gen, and D/G/8 a power of two up to 16 (heads of
 * 8, 16, 32, 64 or 128 channels); DSC_ERROR_NOT_SUPPORTED otherwise. */
dsc_status_t dsc_bwd_gen(const void* x, const void* h, const void* Wg, const void* dy, void* dx, void* dw,
                         int64_t B, int64_t T, int64_t D, int64_t G, int32_t W, int64_t K, int32_t residual,
                         dsc_dtype_t dtype, dsc_stream_t stream);

/* dsc_bwd_gen on packed sequences: pos [B,T] as for dsc_fwd_gen_varlen; a masked
 * tap contributes to neither dx nor dw (its dw is 0). */
dsc_status_t dsc_bwd_gen_varlen(const void* x, const void* h, const void* Wg, const int32_t* pos,
                                const void* dy, void* dx, void* dw, int64_t B, int64_t T, int64_t D,
                                int64_t G, int32_t W, int64_t K, int32_t residual, dsc_dtype_t dtype,
                                dsc_stream_t stream);

/* ---------------------------------------------------------------- decoding
 *
 * Generation appends one token per sequence at a time. The forward definition
 * (Mecanismo) at that token t reads, besides x_t, only the W-1 inputs before it,
 * so each sequence carries them between calls in a ring:
 *     state [B, W-1, D]  input x_s of sequence b sits in slot s mod (W-1);
 *     pos   [B] int32    t = pos[b], the index of row b's incoming token in its
 *                        sequence (0 for its first); negative: an idle row.
 * One step computes, for every row b with t = pos[b] >= 0 and the filter
 * f[b,c,k] of its token,
 *     y[b,c] = residual*x[b,c] + sum_{k=0}^{min(W-1,t)} f[b,c,k] * x_{t-k}[c],
 *              x_t = x[b,:],  x_{t-k} = state[b, (t-k) mod (W-1), :]  (k >= 1),
 * and then stores x[b,:] into slot t mod (W-1), which held x_{t-W+1}: read by
 * this step, by no later one. Slots of steps before 0 are never read, so a new
 * sequence starts without clearing its ring, and rows of one batch may sit at
 * different positions. Idle rows leave y[b,:] and their ring untouched. y equals
 * row t of the forward pass over the whole sequence, up to float32 rounding
 * order. (The page prints no decode step; this is its forward definition taken
 * one step at a time.)
 * Conventions: as above, with x, y [B, D], w [B, G, W], z [B, R] for the one new
 *   token per row. state is read and written (it may overlap no other tensor);
 *   W = 1 keeps no ring and state may then be NULL. pos and len are device
 *   arrays that only need 4-byte alignment; their values are read on the device
 *   and never checked by the host. B == 0 -> DSC_SUCCESS, nothing done.
 *   Every other check is the one of the calls above, in the same order. */

/* Decode step, head-wise filters: f[b,c,k] = w[b, c/Hc, k], Hc = D/G.
 * x [B,D], w [B,G,W], pos [B] in; state [B,W-1,D] in/out; y [B,D] out. */
dsc_status_t dsc_decode_step(const void* x, const void* w, const int32_t* pos, void* state, void* y,
                             int64_t B, int64_t D, int64_t G, int32_t W, int32_t residual,
                             dsc_dtype_t dtype, dsc_stream_t stream);

/* Decode step, low-rank filters: f[b,c,k] = sum_r z[b,r] * U[r, c*W+k], generated
 * on-chip as in dsc_lowrank_fwd. x [B,D], z [B,R], U [R,D*W], pos [B] in;
 * state [B,W-1,D] in/out; y [B,D] out. */
dsc_status_t dsc_lowrank_decode_step(const void* x, const void* z, const void* U, const int32_t* pos,
                                     void* state, void* y, int64_t B, int64_t D, int32_t R, int32_t W,
                                     int32_t residual, dsc_dtype_t dtype, dsc_stream_t stream);

/* The ring after a prompt: row b has consumed the first n = len[b] tokens of
 * x [B,T,D] (n clamped to [0, T] on the device); slot s mod (W-1) of state[b]
 * receives x[b,s,:] for max(0, n-W+1) <= s < n, other slots keep their
 * contents. Decoding then continues with pos[b] = n. x [B,T,D], len [B] in;
 * state [B,W-1,D] in/out. B == 0, T == 0 or W == 1 -> DSC_SUCCESS, nothing done. */
dsc_status_t dsc_decode_state_from_prefill(const void* x, const int32_t* len, void* state, int64_t B,
                                           int64_t T, int64_t D, int32_t W, dsc_dtype_t dtype,
                                           dsc_stream_t stream);

/* A static, human-readable name for a status code (never NULL). */
const char* dsc_status_string(dsc_status_t status);

/* DSC_ABI_VERSION of the built library. */
int32_t dsc_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSC_H_ */
