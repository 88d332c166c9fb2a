/*
 * vsa.h - C ABI of the VSA (Video Sparse Attention) coarse-fine attention
 * operator for one AMD Instinct MI355X (gfx950) GPU.
 *
 * The operator (VSA summary page, paperlayer.ai arXiv 2505.13389, section 2
 * "Methods" and Appendix B "Pseudocode of VSA"; VSA reading notes, key
 * designs 1-3):
 *   1. partition the T x H x W latent into (Ct, Ch, Cw) cubes ((4, 4, 4) by
 *      default), one tile of Bt = Ct*Ch*Cw tokens each (64 by default);
 *   2. mean-pool Q, K, V per cube and run dense attention over the cubes,
 *      giving A_c and O_c;
 *   3. keep the top-K key cubes of every row of A_c (or take caller-supplied
 *      per-query-cube lists of variable length, the VSA2 "variable number of
 *      key-value pairs per query", VSA2 abstract);
 *   4. exact token attention of every query cube over the tokens of its kept
 *      cubes only (O_f);
 *   5. O = O_c (repeated to the cube's tokens) * G_c + O_f * G_f.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Float tensors are [B, heads, T, H, W, head_dim] contiguous (raster token
 *   order, head_dim fastest) in the problem's dtype (fp32 or bf16), unless the
 *   argument says otherwise. Pooled tensors ("_c") are fp32 [B, heads, Nc,
 *   head_dim], cubes in row-major order over (T/Ct, H/Ch, W/Cw); Nc = T*H*W/Bt.
 *   Key blocks (vsa_problem.kcube_*) default to the query cube; when they
 *   differ, keys and values are pooled per key block (k_c, v_c, dk_c, dv_c
 *   are [B, heads, Nk, head_dim], Nk = T*H*W/Bk) while queries, o_c and
 *   lse_c stay per query cube (Nq = Nc rows).
 *   Per-token scalars (LSE_f, delta) are fp32 [B, heads, T, H, W]. With the
 *   TILED layout (vsa_layout below) every token tensor and per-token array of
 *   the problem is cube-major instead ([B, heads, Nc, Bt, ...]): wherever an
 *   argument below says "raster", read "in the problem's token order".
 * - Index lists: idx is int32 [B, heads, Nc, list_stride], len int32
 *   [B, heads, Nc]. Row i holds len[i] strictly increasing key-block ids in
 *   [0, Nk); entries beyond len[i] are ignored.
 * - Every pointer is a device pointer unless documented as host, and must be
 *   16-byte aligned. The caller allocates and owns every buffer; the library
 *   never allocates or frees device memory and keeps no per-call state.
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *   is asynchronous: nothing synchronises unless documented.
 * - Outputs are fully overwritten, never accumulated.
 * - Errors: host-checkable faults return an error before anything is
 *   enqueued; a failed launch returns VSA_ERR_HIP. Nothing aborts or prints.
 *   Invalid index lists (duplicates, out of range, unsorted) are undefined
 *   behaviour unless checked first with vsa_check_lists_host or
 *   vsa_validate_lists.
 */
#ifndef VSA_H
#define VSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VSA_OK = 0,
  VSA_ERR_NULL = 1,        /* a required pointer is NULL                      */
  VSA_ERR_SHAPE = 2,       /* B/heads < 1, T/H/W not positive multiples of the
                              cube sides, an invalid cube side, or a size that
                              overflows                                       */
  VSA_ERR_HEAD_DIM = 3,    /* head_dim not 64 or 128                         */
  VSA_ERR_DTYPE = 4,       /* unknown dtype                                  */
  VSA_ERR_TOPK = 5,        /* topk outside [0, Nk] or list_stride invalid    */
  VSA_ERR_ALIGN = 6,       /* a pointer is not 16-byte aligned               */
  VSA_ERR_WORKSPACE = 7,   /* workspace / saved buffer smaller than required */
  VSA_ERR_INDEX = 8,       /* an index list failed validation                */
  VSA_ERR_UNSUPPORTED = 9, /* valid request this build does not implement (a
                              cube of other than 32 to 256 tokens, a key
                              block of other than 16 to 256, too many cubes),
                              an unknown pool_mode or layout, or in-place
                              tiling                                          */
  VSA_ERR_HIP = 10,        /* a HIP call or kernel launch failed             */
  VSA_ERR_SCALE = 11       /* scale is negative, NaN or infinite             */
} vsa_status;

typedef enum { VSA_F32 = 0, VSA_BF16 = 1 } vsa_dtype;

/* Cube pooling of the coarse stage. MEAN is the method (VSA summary page,
 * section 2 and Appendix B); MAX is the variant its ablation study compares
 * (section 3, Experiments): the per-channel maximum over a cube, whose
 * gradient goes to the first maximum in cube order. */
typedef enum { VSA_POOL_MEAN = 0, VSA_POOL_MAX = 1 } vsa_pool_mode;

/* Token order of every token tensor of a problem (q, k, v, gates, o, d_o,
 * gradients, O_f, and the per-token fp32 arrays LSE_f / delta). RASTER is
 * [B, heads, T, H, W, ...]; TILED is cube-major [B, heads, Nc, Bt, ...] with
 * token l of cube c at position Bt*c + l, the tiled sequence of the VSA
 * summary page's pseudocode (Appendix B), which tiles before the attention
 * layer and untiles after it, so a model can keep activations tiled across
 * layers (vsa_tile / vsa_untile convert). Index lists and pooled tensors do
 * not depend on it. */
typedef enum { VSA_LAYOUT_RASTER = 0, VSA_LAYOUT_TILED = 1 } vsa_layout;

typedef struct {
  int32_t B, heads;      /* batch and heads; every (b, h) is independent      */
  int32_t T, H, W;       /* latent grid, multiples of the cube sides           */
  int32_t head_dim;      /* 64 or 128                                          */
  int32_t dtype;         /* vsa_dtype of every float tensor except pooled ones */
  float scale;           /* softmax scale of both stages; 0 => 1/sqrt(head_dim) */
  int32_t topk;          /* > 0: keep the K best key blocks per query cube
                            (1..Nk); 0: the caller supplies the lists          */
  int32_t list_stride;   /* row stride of idx; 0 => topk. Top-K mode needs
                            list_stride >= topk; list mode needs 1..Nk         */
  int32_t pool_mode;     /* vsa_pool_mode; 0 = mean                            */
  int32_t layout;        /* vsa_layout; 0 = raster                             */
  int32_t cube_t, cube_h, cube_w;
                         /* cube sides (Ct, Ch, Cw); 0 => 4. The VSA summary
                            page (section 2 "Methods") names the cube
                            (Ct, Ch, Cw) with tile size Bt = Ct*Ch*Cw and
                            weighs tile sizes in its design exploration.
                            Each side a power of two, Cw >= 4, Bt in
                            {32, 64, 128, 256}. In-cube token order is
                            row-major (t', y', x'). The fine kernels take a
                            256-token cube as its two 128-token halves (split
                            along its first side longer than 1); pooling, the
                            coarse stage and the lists stay per cube.         */
  int32_t kcube_t, kcube_h, kcube_w;
                         /* sides of the key blocks; all 0 => the query cube.
                            The same page's tile-size exploration compares
                            query and key tiles of different sizes (Bq x Bk
                            blocks, such as 64 x 16): keys and values are
                            tiled and pooled by this shape, the coarse scores
                            are Nq x Nk (Nq = N/Bt query cubes, Nk = N/Bk key
                            blocks), index lists name key blocks, and topk /
                            list_stride range over 1..Nk. Powers of two,
                            kcube_w >= 4, Bk in {16, 32, 64, 128, 256}
                            (16-token blocks are taken two at a time by the
                            fine kernels, 256-token blocks as two halves).
                            The tiled layout needs kcube = cube.            */
} vsa_problem;

/* Short text for a status code (static storage, never NULL). */
const char* vsa_status_string(vsa_status s);

/* Library version as major*10000 + minor*100 + patch. */
int32_t vsa_version(void);

/* Largest Nc or Nk (cubes or key blocks per (b, h)) the coarse stage
 * accepts in this build (8192). */
int32_t vsa_max_cubes(void);

/* Bytes of device workspace vsa_forward (training = 0) or vsa_backward
 * (training = 1) needs for problem p; 0 if p is invalid. The workspace holds
 * scratch only (the coarse logits, fp32 Nc x Nk per (b, h), the processing
 * orders, and for the backward the coarse softmax and its gradient, d_o_f,
 * delta, the transposed lists and their bitmask); its contents are
 * meaningless between calls. */
size_t vsa_workspace_bytes(const vsa_problem* p, int32_t training);

/* Bytes of the `saved` buffer a training forward fills and vsa_backward
 * reads. 0 if p is invalid. Layout, each region starting on a 256-byte
 * boundary of the buffer: Q_c, K_c, V_c, O_c (fp32 [B, heads, Nc or Nk,
 * head_dim] each), LSE_c (fp32 [B, heads, Nc]), LSE_f (fp32 [B, heads, T, H,
 * W]), O_f (dtype, raster). */
size_t vsa_saved_bytes(const vsa_problem* p);

/* Whole forward, steps 1-5 above.
 *   q, k, v     : inputs (dtype, raster).
 *   g_c, g_f    : gates, shaped like o (dtype). NULL means the gate is all
 *                 ones (an ungated branch, as when the fine gate is removed at
 *                 the start of sparse adaptation; reading notes key design 5).
 *   idx, len    : topk > 0: outputs, the ascending top-K lists (len = K);
 *                 topk == 0: inputs, the caller's lists.
 *   o           : output (dtype, raster).
 *   saved       : NULL for inference; otherwise vsa_saved_bytes(p) bytes that
 *                 vsa_backward will read.
 *   workspace   : ws_bytes >= vsa_workspace_bytes(p, 0) bytes. */
vsa_status vsa_forward(const vsa_problem* p, const void* q, const void* k, const void* v,
                       const void* g_c, const void* g_f, int32_t* idx, int32_t* len,
                       void* o, void* saved, void* workspace, size_t ws_bytes, void* stream);

/* Whole backward of sum(O * dO) with the selection held constant (the top-K
 * mask is piecewise constant and carries no gradient). The method is trained
 * end to end as one differentiable operator, the gate letting the learned
 * coarse and fine branches both receive gradient (VSA summary page,
 * Abstract, and section 1 "Introduction", the gated combination): this entry
 * point returns the gradients of both branches, the coarse one through the
 * pooling into every token of a cube. Inputs as for the
 * forward that filled `saved` (same q, k, v, g_c, g_f, idx, len), d_o
 * (dtype, raster). Outputs dq, dk, dv (dtype, raster) and dg_c, dg_f (dtype,
 * raster; each may be NULL when its gate was NULL, then it is not written).
 * workspace: ws_bytes >= vsa_workspace_bytes(p, 1). Both dtypes: bf16 runs
 * the MFMA kernels, fp32 a one-thread-per-token path in fp32 arithmetic. */
vsa_status vsa_backward(const vsa_problem* p, const void* q, const void* k, const void* v,
                        const void* g_c, const void* g_f, const int32_t* idx, const int32_t* len,
                        const void* saved, const void* d_o, void* dq, void* dk, void* dv,
                        void* dg_c, void* dg_f, void* workspace, size_t ws_bytes, void* stream);

/* ---- stage-level entry points (same conventions; for per-stage parity and
 * timing; vsa_forward / vsa_backward chain exactly these kernels) ---------- */

/* Step 1, cube mean-pool: q_c (fp32 [B, heads, Nc, head_dim]) and k_c/v_c
 * (fp32 [B, heads, Nk, head_dim]) are the means of the tokens of every cube
 * or key block (VSA summary page, Appendix B;
 * reading notes key design 1), or their per-channel maxima when pool_mode
 * is VSA_POOL_MAX. */
vsa_status vsa_pool(const vsa_problem* p, const void* q, const void* k, const void* v,
                    float* q_c, float* k_c, float* v_c, void* stream);

/* Steps 2-3, coarse stage: S_c = scale * Q_c K_c^T, A_c = row softmax,
 * o_c = A_c V_c (fp32 [B, heads, Nc, head_dim]) and lse_c = log-sum-exp of
 * each row of S_c (fp32 [B, heads, Nc]). With topk > 0 it also writes idx /
 * len: per row the K largest logits (ties to the smaller key-block id) as an
 * ascending list (VSA summary page, section 2 and Appendix B; reading notes
 * key design 1, and the fused softmax + top-K + mask-to-index kernel of the
 * notes' training section). With topk == 0 idx / len are not touched (may be
 * NULL). S_c (fp32, Nc x Nk per (b, h)) lives in the workspace
 * (ws_bytes >= vsa_workspace_bytes(p, 0)). Requires Nc, Nk <= vsa_max_cubes().
 * The logits, LSE and selection are computed in fp32; for bf16 problems the
 * product A_c V_c runs on bf16 matrix cores with each fp32 operand split into
 * a bf16 head and tail (relative error at most 3 * 2^-16 per term). */
vsa_status vsa_coarse(const vsa_problem* p, const float* q_c, const float* k_c, const float* v_c,
                      float* o_c, float* lse_c, int32_t* idx, int32_t* len, void* workspace,
                      size_t ws_bytes, void* stream);

/* Step 4, fine block-sparse attention: for every query token of cube i,
 * softmax attention over the tokens of the key blocks listed in row i only
 * (VSA summary page, section 2 "Fine stage" and Appendix B; reading notes key
 * design 2). o_f (dtype, raster) and lse_f (fp32 [B, heads, T, H, W]); an
 * empty list gives o_f = 0 and lse_f = -inf. For bf16, the workspace
 * (ws_bytes >= vsa_workspace_bytes(p, 0)) holds the query-cube processing
 * order; fp32 problems need none (may be NULL). */
vsa_status vsa_fine_forward(const vsa_problem* p, const void* q, const void* k, const void* v,
                            const int32_t* idx, const int32_t* len, void* o_f, float* lse_f,
                            const void* workspace, size_t ws_bytes, void* stream);

/* Steps 4 and 5 fused, the kernel vsa_forward runs: the fine stage with the
 * gated combine in its epilogue, o = O_c[cube] * g_c + O_f * g_f (dtype,
 * raster), so O_f never goes to memory unless o_f is given. o_f (dtype,
 * raster) and lse_f (fp32) are optional outputs (NULL = not written); O_f is
 * rounded to the dtype before the combine, so o equals vsa_combine of the
 * returned o_f. Gates NULL => ones. Workspace as for vsa_fine_forward. */
vsa_status vsa_fine_combine(const vsa_problem* p, const void* q, const void* k, const void* v,
                            const int32_t* idx, const int32_t* len, const float* o_c,
                            const void* g_c, const void* g_f, void* o, void* o_f, float* lse_f,
                            const void* workspace, size_t ws_bytes, void* stream);

/* vsa_fine_combine without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). It runs the same kernels; the query-cube
 * order they need lives in a 4 MiB device array inside the library (one per
 * GPU, held until the process ends), so B * heads * Nc may not exceed
 * 1,048,576 (VSA_ERR_WORKSPACE otherwise, before anything is enqueued). The
 * call allocates nothing. Problems with 256-token cubes or key blocks are
 * refused (VSA_ERR_UNSUPPORTED: their expanded lists need a workspace). It
 * uses the array of the current device, so
 * `stream` must belong to the current device; the first call on a device
 * looks up the array's address (VSA_ERR_HIP if that fails). Every call on a
 * GPU shares that GPU's array: calls that overlap on one GPU (other streams,
 * other threads) race and must be serialised by the caller; consecutive calls
 * on one stream are safe. Arguments and results as for vsa_fine_combine. */
vsa_status vsa_fine_combine_noalloc(const vsa_problem* p, const void* q, const void* k, const void* v,
                                    const int32_t* idx, const int32_t* len, const float* o_c, const void* g_c,
                                    const void* g_f, void* o, void* o_f, float* lse_f, void* stream);

/* Step 5, gated combine + untile: o = O_c[cube(token)] * g_c + o_f * g_f
 * (reading notes key design 3; App. B repeat of the coarse output). Gates
 * NULL => ones. */
vsa_status vsa_combine(const vsa_problem* p, const float* o_c, const void* o_f,
                       const void* g_c, const void* g_f, void* o, void* stream);

/* Backward of step 5 (calculus of the combine): dg_c = dO * O_c[cube],
 * dg_f = dO * O_f, d_o_f = dO * G_f (dtype, raster), delta = rowsum(d_o_f *
 * o_f) (fp32 [B, heads, T, H, W]) and d_o_c[c] = sum over the Bt tokens of
 * cube c of dO * G_c (fp32 [B, heads, Nc, head_dim]). dg_c / dg_f may be
 * NULL (not written). */
vsa_status vsa_combine_backward(const vsa_problem* p, const void* d_o, const float* o_c,
                                const void* o_f, const void* g_c, const void* g_f,
                                void* dg_c, void* dg_f, void* d_o_f, float* delta, float* d_o_c,
                                void* stream);

/* Index transpose for the backward: k2q_off int32 [B, heads, Nk + 1] and
 * k2q int32 [B, heads, Nc * list_stride]: for key block j the query cubes i
 * whose list holds j, ascending, at k2q[(b,h) * Nc * list_stride +
 * k2q_off[(b,h)][j] ... k2q_off[(b,h)][j+1]). Uses a bitmask in the
 * workspace (ws_bytes >= vsa_workspace_bytes(p, 1)). */
vsa_status vsa_index_transpose(const vsa_problem* p, const int32_t* idx, const int32_t* len,
                               int32_t* k2q_off, int32_t* k2q, void* workspace, size_t ws_bytes,
                               void* stream);

/* Backward of step 4 and of the pooling: dq, dk, dv (dtype, raster) =
 * fine-attention gradient + (dq_c, dk_c, dv_c)[cube or key block] / its
 * token count (with max pooling the pooled gradient goes to the argmax token
 * instead), where the pooled gradients (fp32 [B, heads, Nc or Nk, head_dim])
 * come from vsa_coarse_backward.
 * lse_f from the forward; d_o_f and delta from vsa_combine_backward
 * (workspace: ws_bytes >= vsa_workspace_bytes(p, 1)); k2q_off / k2q from
 * vsa_index_transpose. bf16 or fp32. dQ walks each query cube's list, dK / dV
 * walk the transposed lists, so no atomics are used and the result is
 * deterministic. With 256-token cubes or key blocks the kernels run on their
 * 128-token halves and build the halves' transposed lists in the workspace
 * themselves (k2q_off / k2q must still be valid pointers; they are not read). */
vsa_status vsa_fine_backward(const vsa_problem* p, const void* q, const void* k, const void* v,
                             const int32_t* idx, const int32_t* len, const int32_t* k2q_off,
                             const int32_t* k2q, const float* lse_f, const void* d_o_f,
                             const float* delta, const float* dq_c, const float* dk_c,
                             const float* dv_c, void* dq, void* dk, void* dv, void* workspace,
                             size_t ws_bytes, void* stream);

/* Backward of steps 1-2 at cube level (dense attention backward in fp32):
 * dq_c (Nc rows), dk_c, dv_c (Nk rows) (fp32 [B, heads, rows, head_dim])
 * from q_c, k_c, v_c, o_c,
 * lse_c and d_o_c. workspace >= vsa_workspace_bytes(p, 1). */
vsa_status vsa_coarse_backward(const vsa_problem* p, const float* q_c, const float* k_c,
                               const float* v_c, const float* o_c, const float* lse_c,
                               const float* d_o_c, float* dq_c, float* dk_c, float* dv_c,
                               void* workspace, size_t ws_bytes, void* stream);

/* ---- list validation ----------------------------------------------------- */

/* Token-order conversion: xt (cube-major [B, heads, Nc, Bt, head_dim]) from
 * x (raster [B, heads, T, H, W, head_dim]) and back, both in the problem's
 * dtype; the problem's layout field is ignored. Not in place (x != xt). */
vsa_status vsa_tile(const vsa_problem* p, const void* x, void* xt, void* stream);
vsa_status vsa_untile(const vsa_problem* p, const void* xt, void* x, void* stream);

/* Latents whose sides are not multiples of the cube's. The VSA summary page
 * (paperlayer.ai, arXiv 2505.13389), section 5 "Limitation and Conclusion",
 * notes that (4, 4, 4) cubes need sides divisible by 4 and names the remedy:
 * generate a slightly larger latent and crop the result.
 *
 * vsa_compatible_latent: the smallest grid Tc x Hc x Wc with every side a
 * multiple of the matching cube side (ct, ch, cw; 0 => 4) that contains
 * T x H x W (each side rounded up). Host only; VSA_ERR_NULL for a NULL output
 * pointer, VSA_ERR_SHAPE for a side <= 0, a cube side that is not a power of
 * two, or a result that would overflow int32. */
vsa_status vsa_compatible_latent(int32_t T, int32_t H, int32_t W, int32_t ct, int32_t ch, int32_t cw, int32_t* Tc,
                                 int32_t* Hc, int32_t* Wc);

/* vsa_crop: out = the leading T x H x W region of x, a token tensor of the
 * (compatible) problem p in p's layout, written in raster order
 * [B, heads, T, H, W, head_dim], p's dtype. From the tiled layout this is the
 * untile and the crop in one pass.
 * vsa_pad: the reverse embedding. out, a token tensor of p in p's layout,
 * takes x (raster [B, heads, T, H, W, head_dim]) at the origin and zeros at
 * every token outside it.
 * Both need 1 <= T <= p->T, 1 <= H <= p->H, 1 <= W <= p->W (else
 * VSA_ERR_SHAPE), 16-byte aligned non-NULL pointers and x != out
 * (VSA_ERR_UNSUPPORTED); asynchronous on `stream`. */
vsa_status vsa_crop(const vsa_problem* p, const void* x, int32_t T, int32_t H, int32_t W, void* out, void* stream);
vsa_status vsa_pad(const vsa_problem* p, const void* x, int32_t T, int32_t H, int32_t W, void* out, void* stream);

/* Host check of explicit lists (host pointers): every len in [0, list_stride],
 * every listed id in [0, Nk), strictly increasing. Returns VSA_OK or
 * VSA_ERR_INDEX. Runs on the CPU only. */
vsa_status vsa_check_lists_host(const vsa_problem* p, const int32_t* idx, const int32_t* len);

/* The same check on device lists; synchronises `stream` to read the verdict.
 * `flag` is a caller-provided device int32 used as the result cell. */
vsa_status vsa_validate_lists(const vsa_problem* p, const int32_t* idx, const int32_t* len,
                              int32_t* flag, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VSA_H */
