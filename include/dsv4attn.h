/*
 * dsv4attn.h - C ABI of the MI355X (gfx950) DeepSeek-V4 hybrid attention core.
 *
 * The operations follow the Hugging Face Transformers model page "DeepSeek-V4":
 *   "Hybrid attention (§2.3)"  - CSA (compressed pool at rate m with overlapping windows,
 *                                then the Lightning Indexer's top-k), HCA (pool at rate m'
 *                                with disjoint windows, every entry attended), and the shared
 *                                skeleton: one K=V head, interleaved partial RoPE on the
 *                                trailing qk_rope_head_dim channels, output rotation at
 *                                position -i (eq. 26), per-head sink (eq. 27), and the
 *                                sliding-window K=V branch concatenated before the pool.
 *   "Attention mask layout"    - which keys each query sees (window cut, -1 sentinel,
 *                                entry w visible iff w < (t+1)//m).
 *   "DeepseekV4Config"         - field meanings (head_dim, sliding_window, index_topk ...).
 * The page names eqs. 13-17, 26, 27 without printing them; the exact forms used here are
 * the readings listed beside each function.
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a DEVICE pointer unless stated otherwise; the caller owns
 *     all buffers.  The library never allocates or frees device memory; scratch memory is
 *     passed in explicitly (csa_index_topk's workspace), except for the fixed static array
 *     of csa_index_topk_noalloc.
 *   - stream is a hipStream_t (NULL = the default stream).  Calls only enqueue work and
 *     return; results are ready when the stream reaches them.
 *   - Tensors are dense row-major with the channel axis innermost.  dtype DSV4_FP32 or
 *     DSV4_BF16 applies to the activation tensors (q, kv, gate, pools, windows, outputs);
 *     slot biases, sinks, indexer weights and scores are always float32; indices int32.
 *   - Positions: every query / token / entry has a sequence index (its row in the
 *     sequence); its RoPE position is that index plus rope_pos_offset.  Visibility always
 *     uses sequence indices.  RoPE (reading R10): pair i of the trailing r channels is
 *     (C-r+2i, C-r+2i+1), frequency rope_theta^(-2i/r), angle = position * frequency,
 *     angles evaluated in double precision.
 *   - Return value: DSV4_OK, or an error code.  Arguments are validated before any work is
 *     enqueued; on error nothing is launched and dsv4_last_error() (per calling thread)
 *     describes the problem.  DSV4_ERR_LAUNCH reports a failed kernel launch.
 *   - Index arguments read on the device (topk_idx) are bounds-checked by the kernels:
 *     any value outside [0, N_cap) is treated as the -1 sentinel.
 */
#ifndef DSV4ATTN_H
#define DSV4ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSV4_ABI_VERSION 1

enum dsv4_dtype { DSV4_FP32 = 0, DSV4_BF16 = 1 };

enum dsv4_status {
  DSV4_OK = 0,
  DSV4_ERR_INVALID = 1,     /* null required pointer, bad or inconsistent sizes         */
  DSV4_ERR_UNSUPPORTED = 2, /* valid request outside what the compiled kernels cover     */
  DSV4_ERR_LAUNCH = 3,      /* the HIP runtime rejected a kernel launch                  */
  DSV4_ERR_WORKSPACE = 4    /* workspace pointer NULL or smaller than required           */
};

int dsv4_abi_version(void);
const char* dsv4_status_string(int status);
/* Detail of the last error returned on the calling thread ("" if none). */
const char* dsv4_last_error(void);

/*
 * csa_compress - pool tokens into compressed KV entries ("Hybrid attention (§2.3)", CSA and
 * HCA items; "Attention mask layout", HCA paragraph for the window of an entry).
 *
 * Reading R1/R2/R5: for each entry w in [entry_begin, entry_end) and channel c,
 *   window(w) = tokens [(w-1)m, (w+1)m) if overlap (CSA, 2m slots) else [w m, (w+1) m)
 *               (HCA, m slots); slot s = token - window start; tokens before 0 are absent
 *               and excluded from the softmax;
 *   a_j       = gate[b,j,c] + bias[s,c]            (bias NULL: zero)
 *   pool[b,w,c] = sum_j softmax_j(a)_j * x[b,j,c]
 *   then channels [C-rope_dim, C) are rotated at position (w+1)m - 1 + rope_pos_offset.
 *
 *   x, gate : [B, S, C] dtype.   bias : [overlap ? 2m : m, C] float32 or NULL.
 *   pool    : [B, N_cap, C] dtype; rows [entry_begin, entry_end) are written, others kept.
 *   Requires 0 <= entry_begin <= entry_end <= N_cap, entry_end * m <= S (every window is
 *   closed), C even, rope_dim even and <= min(C, 256), m >= 1 (DSV4_ERR_INVALID otherwise).
 *   C must be a multiple of 8 up to 2048, or any even C up to 512 (DSV4_ERR_UNSUPPORTED
 *   otherwise).  Pointers 16-byte aligned.
 */
int csa_compress(const void* x, const void* gate, const float* bias, void* pool, int B, int S,
                 int C, int m, int overlap, int entry_begin, int entry_end, int N_cap,
                 int rope_dim, double rope_theta, long long rope_pos_offset, int dtype,
                 void* stream);

/*
 * compressor_cache_update - one decode step of a compressor cache ("Cache layers": the HCA
 * cache's compressor buffer / pool / count, the CSA cache's compressor with its overlap
 * state and the parallel indexer's buffer / pool / count / overlap at index_head_dim).
 *
 * Sequence b has L = lengths[b] tokens including the new one (L >= 1; L < 1: untouched).
 * Its raw token ring x_ring[b] / gate_ring[b] holds the last span tokens, span = 2m with
 * overlap (CSA) or m (HCA): token position p lives in slot p mod span.  The call stores the
 * new token (x_new[b], gate_new[b]) in slot (L-1) mod span; when emit != 0 and L mod m == 0
 * the token closes entry w = L/m - 1, which is pooled from the ring exactly as csa_compress
 * defines it (same window, bias and RoPE at (w+1)m - 1 + rope_pos_offset) and written to
 * pool[b, w] (entries w >= N_cap are not written).  emit = 0 only fills the ring (e.g. with
 * the last span tokens of a prefill whose entries are already pooled).
 *
 *   x_new, gate_new : [B, C] dtype.  x_ring, gate_ring : [B, span, C] dtype (caller-owned
 *   state, kept across calls).  bias : [span, C] float32 or NULL.  pool : [B, N_cap, C].
 *   lengths : [B] int32 device array.  C, rope_dim and alignment as for csa_compress;
 *   span <= 4096 (DSV4_ERR_UNSUPPORTED otherwise).  Sequences are independent; one call
 *   per layer and per compressor (the CSA K=V pool and its indexer keys are two calls).
 */
int compressor_cache_update(const void* x_new, const void* gate_new, void* x_ring,
                            void* gate_ring, const float* bias, void* pool, const int* lengths,
                            int B, int C, int m, int overlap, int N_cap, int rope_dim,
                            double rope_theta, long long rope_pos_offset, int emit, int dtype,
                            void* stream);

/*
 * compressor_cache_update_pair - two compressor_cache_update calls in one launch, for the two
 * compressors of one layer that share lengths, m, overlap and N_cap ("Cache layers": the CSA
 * cache's compressor and the parallel indexer's).  Compressor 1 is (x_new, gate_new, x_ring,
 * gate_ring, bias, pool, C, rope_dim), compressor 2 the same with suffix 2; each exactly as
 * compressor_cache_update defines it, with the same argument rules (both must pass them,
 * else nothing is launched).  The two compressors' buffers must not overlap.
 */
int compressor_cache_update_pair(const void* x_new, const void* gate_new, void* x_ring, void* gate_ring,
                                 const float* bias, void* pool, int C, int rope_dim, const void* x2_new,
                                 const void* gate2_new, void* x2_ring, void* gate2_ring, const float* bias2,
                                 void* pool2, int C2, int rope_dim2, const int* lengths, int B, int m, int overlap,
                                 int N_cap, double rope_theta, long long rope_pos_offset, int emit, int dtype,
                                 void* stream);

/*
 * csa_compress_split - csa_compress with separate projections for the two halves of each
 * overlapping window (reading R4b of the CSA compressor: the earlier half of entry w's window,
 * tokens (w-1)m .. wm-1, takes its values and gates from x_prev / gate_prev, the later half,
 * wm .. (w+1)m-1, from x / gate; one softmax spans all 2m slots).  Always overlapping.
 *
 *   x_prev, gate_prev : [B, S, C] dtype, both given or both NULL (NULL = csa_compress with
 *     overlap = 1).  Every other argument as csa_compress.
 */
int csa_compress_split(const void* x, const void* gate, const void* x_prev, const void* gate_prev,
                       const float* bias, void* pool, int B, int S, int C, int m, int entry_begin,
                       int entry_end, int N_cap, int rope_dim, double rope_theta,
                       long long rope_pos_offset, int dtype, void* stream);

/*
 * compressor_cache_update_split - compressor_cache_update for the R4b compressor (overlapping
 * windows, separate projections for the two halves): the new token's second projection
 * (x_prev_new, gate_prev_new [B, C]) goes into its own rings (x_prev_ring, gate_prev_ring
 * [B, 2m, C], slot (L-1) mod 2m like the first), and a closing entry pools its earlier half
 * from them.  All four second-projection pointers are required; the rest as
 * compressor_cache_update with overlap = 1.
 */
int compressor_cache_update_split(const void* x_new, const void* gate_new, const void* x_prev_new,
                                  const void* gate_prev_new, void* x_ring, void* gate_ring,
                                  void* x_prev_ring, void* gate_prev_ring, const float* bias,
                                  void* pool, const int* lengths, int B, int C, int m, int N_cap,
                                  int rope_dim, double rope_theta, long long rope_pos_offset,
                                  int emit, int dtype, void* stream);

/*
 * csa_index_topk - Lightning Indexer scores and top-k per query ("Hybrid attention (§2.3)",
 * CSA item, eqs. 13-17; "Attention mask layout", CSA paragraph for the -1 sentinel;
 * "DeepseekV4Config": index_n_heads, index_head_dim, index_topk).
 *
 * Query t of sequence b has sequence index q_pos0[b] + t and V = min((q_pos0[b]+t+1)//m,
 * n_pool[b]) candidate entries (reading R7).  Reading R8:
 *   score[w] = sum_h w_idx[b,t,h] * max(0, sum_c q_idx[b,t,h,c] * k_pool[b,w,c]),  w < V.
 * Reading R9: the min(k, V) largest scores are kept; equal scores keep the lower entry
 * index; -0.0 ranks as +0.0.  topk_idx[b,t,:] lists the kept entries in ascending index
 * order, then -1 in the remaining slots; topk_score (optional) holds their scores (and 0
 * beside each -1; a kept score of -0.0 may be reported as +0.0).
 *
 *   q_idx   : [B, T, nI, cI] dtype.  w_idx : [B, T, nI] float32.
 *   k_pool  : [B, N_cap, cI] dtype (the indexer's own compressed keys, not rotated).
 *   q_pos0, n_pool : [B] int32 device arrays.
 *   topk_idx: [B, T, k] int32 out.  topk_score: [B, T, k] float32 out, or NULL.
 *   workspace: device scratch of at least csa_index_topk_workspace_size(...) bytes; its
 *   contents are overwritten.
 *   Requires k >= 1, k <= N_cap, k <= 4096, N_cap <= 1<<20.
 */
size_t csa_index_topk_workspace_size(int B, int T, int N_cap, int k);
int csa_index_topk(const void* q_idx, const float* w_idx, const void* k_pool, const int* q_pos0,
                   const int* n_pool, int* topk_idx, float* topk_score, int B, int T, int nI,
                   int cI, int N_cap, int m, int k, void* workspace, size_t workspace_bytes,
                   int dtype, void* stream);

/*
 * csa_index_topk_noalloc - csa_index_topk for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, results and errors as csa_index_topk, without the workspace: the score
 * scratch is a static device array of DSV4_NOALLOC_SCRATCH_BYTES (32 MiB) inside the library,
 * one copy per GPU the library runs on, held until the process ends.  The call allocates and
 * frees nothing.  Requests whose scratch, csa_index_topk_workspace_size(B, T, N_cap, k), exceeds
 * that size return DSV4_ERR_UNSUPPORTED before anything is enqueued (for example 64 decode
 * queries over 32768 entries, 8 MiB, fit; a 4096-query prefill chunk over 8192 entries does not).  All calls on one
 * GPU share its array: calls that overlap in time on one GPU (unordered streams or threads)
 * race and must be serialised by the caller; stream-ordered calls are safe.
 */
#define DSV4_NOALLOC_SCRATCH_BYTES (32u << 20)
int csa_index_topk_noalloc(const void* q_idx, const float* w_idx, const void* k_pool,
                           const int* q_pos0, const int* n_pool, int* topk_idx, float* topk_score,
                           int B, int T, int nI, int cI, int N_cap, int m, int k, int dtype,
                           void* stream);

/*
 * swa_concat - rotate raw K=V rows into the sliding-window buffer ("Hybrid attention
 * (§2.3)", sliding-window K=V branch and partial RoPE items).  Row i of kv_raw[b] is the
 * token at sequence index new_pos0[b] + i; it is rotated at that index + rope_pos_offset
 * and written to kv_win[b, new_pos0[b] + i - kv_pos0[b]] (rows outside [0, S_cap) are
 * skipped).  The window buffer then feeds the attention calls, whose key order is
 * [window rows || compressed entries].  kv_raw may alias kv_win when the rows coincide.
 *
 *   kv_raw : [B, S_new, D] dtype.  kv_win : [B, S_cap, D] dtype.
 *   kv_pos0, new_pos0 : [B] int32 device arrays.  D even, rope_dim even and <= D.
 *   B * S_new * D below 2^32 (DSV4_ERR_UNSUPPORTED otherwise).
 */
int swa_concat(const void* kv_raw, void* kv_win, const int* kv_pos0, const int* new_pos0, int B,
               int S_new, int S_cap, int D, int rope_dim, double rope_theta,
               long long rope_pos_offset, int dtype, void* stream);

/*
 * attend_workspace_size - bytes of the optional workspace of csa_attend / hca_attend for B*T
 * queries of H heads x D channels on the current device; 0 when the split path does not
 * apply (many queries, or a shape outside the bf16 64 x 512 path), in which case NULL is fine.
 */
size_t attend_workspace_size(int B, int T, int H, int D);

/*
 * csa_attend - CSA core attention over [window || selected entries] ("Hybrid attention
 * (§2.3)", shared skeleton; "Attention mask layout", CSA paragraph).
 *
 * For query t of sequence b at sequence index p = q_pos0[b] + t, the keys are the window
 * rows for sequence indices max(0, p-window+1) .. p (reading R11; row = index - kv_pos0[b],
 * rows outside [0, S_kv) are skipped) followed by pool rows topk_idx[b,t,i] for every
 * valid slot i.  Key = value = that (already rotated) row (R15).  With q_rot = q rotated
 * at p + rope_pos_offset (R10) and z_x = scale * <q_rot[h], key_x> (R12):
 *   o[h] = sum_x e^{z_x} key_x / (e^{sink[h]} + sum_x e^{z_x})          (eq. 27, R13)
 *   out[b,t,h] = o[h] with channels [D-rope_dim, D) rotated at -(p + rope_pos_offset)
 *                                                                         (eq. 26, R16)
 *   q   : [B, T, H, D] dtype, not rotated.  kv_win : [B, S_kv, D] dtype, rotated.
 *   pool: [B, N_cap, D] dtype, rotated.  topk_idx : [B, T, k] int32.  sink : [H] float32.
 *   kv_pos0, q_pos0 : [B] int32 device arrays.  out : [B, T, H, D] dtype.
 *   scale <= 0 selects 1/sqrt(D).  Requires window >= 1, D even, rope_dim even <= D.
 *   workspace : NULL, or caller-owned device scratch of at least
 *     attend_workspace_size(B, T, H, D) bytes (16-byte aligned; DSV4_ERR_WORKSPACE when
 *     smaller).  With it, batches of few queries (decode) cut each query's keys into
 *     ranges attended by separate workgroups and merged afterwards; the result is the same
 *     up to fp32 rounding order.  Its contents are scratch between calls.
 */
int csa_attend(const void* q, const void* kv_win, const int* kv_pos0, int S_kv, const void* pool,
               int N_cap, const int* topk_idx, int k, const float* sink, const int* q_pos0,
               void* out, int B, int T, int H, int D, int window, int rope_dim,
               double rope_theta, long long rope_pos_offset, float scale, void* workspace,
               size_t workspace_bytes, int dtype, void* stream);

/*
 * hca_attend - HCA core attention over [window || every visible entry] ("Hybrid attention
 * (§2.3)", HCA item: no indexer, every pool entry contributes; "Attention mask layout",
 * HCA paragraph: entry w is visible to the query at sequence index p iff w < (p+1)//m_hca).
 * Also the sliding-only layer type: pass N_cap = 0 and pool = NULL.
 *
 * Identical to csa_attend except that the compressed keys of query p are pool rows
 * 0 .. min((p+1)//m_hca, n_pool[b]) - 1 (n_pool NULL: N_cap).
 *   pool : [B, N_cap, D] dtype or NULL when N_cap == 0.  n_pool : [B] int32 or NULL.
 */
int hca_attend(const void* q, const void* kv_win, const int* kv_pos0, int S_kv, const void* pool,
               int N_cap, const int* n_pool, int m_hca, const float* sink, const int* q_pos0,
               void* out, int B, int T, int H, int D, int window, int rope_dim,
               double rope_theta, long long rope_pos_offset, float scale, void* workspace,
               size_t workspace_bytes, int dtype, void* stream);

/*
 * hca_attend_pairs - hca_attend (same keys, same result up to fp32 rounding order) computed
 * by the query-pair kernel: two consecutive queries of a sequence share every 32-key tile,
 * which is read from LDS by 2 x 64 query-head rows ("Attention mask layout", HCA paragraph:
 * neighbouring queries see the same entries and all but one window row each).  Covers bf16,
 * H = 64, D = 512, rope_dim 0 or 64 (DSV4_ERR_UNSUPPORTED otherwise); no workspace.  On
 * gfx950 at these shapes hca_attend is faster: each of the pair kernel's four waves must issue
 * its share of the key-row copies itself, and a wave stalls ~200 cycles per 1 KB copy it issues.
 */
int hca_attend_pairs(const void* q, const void* kv_win, const int* kv_pos0, int S_kv, const void* pool,
                     int N_cap, const int* n_pool, int m_hca, const float* sink, const int* q_pos0,
                     void* out, int B, int T, int H, int D, int window, int rope_dim,
                     double rope_theta, long long rope_pos_offset, float scale, int dtype,
                     void* stream);

/*
 * grouped_out_proj - grouped low-rank output projection ("Hybrid attention (§2.3)", grouped
 * output projection item; "DeepseekV4Config": o_groups, o_lora_rank, hidden_size).  Reading:
 * head group g is the run of H/groups consecutive heads; its concatenated outputs
 * (H/groups * D values) times its own [rank, H/groups * D] matrix give the group's rank
 * vector (o_a_proj, a grouped linear); the groups' vectors, concatenated in group order,
 * times the [hidden, groups * rank] matrix give the output (o_b_proj).  No bias.
 *
 *   attn : [T, H, D] dtype (the attention output).  w_a : [groups, rank, H/groups * D].
 *   w_b  : [hidden, groups * rank].  Weights use a linear layer's [out, in] layout.
 *   mid  : caller-owned [T, groups * rank] dtype buffer for the intermediate (written).
 *   out  : [T, hidden] dtype.  Accumulation is fp32; mid is stored in dtype.
 *   groups must divide H.  Every [T, .] operand below 2 GiB (DSV4_ERR_UNSUPPORTED beyond).
 *   bf16 with rank and hidden multiples of 32 and H/groups * D, groups * rank multiples of 64
 *   runs on the MFMA path; other shapes run a plain kernel (same results up to rounding order).
 */
int grouped_out_proj(const void* attn, const void* w_a, const void* w_b, void* mid, void* out, int T,
                     int H, int D, int groups, int rank, int hidden, int dtype, void* stream);

/*
 * linear_bt - y = x . w^T, the dense product behind the projections around the attention core
 * (the factors of the grouped output projection above; the upstream projections that feed the
 * indexer and the attention are products of the same form).
 *
 *   x : [M, K] dtype.  w : [N, K] dtype (a linear layer's [out, in] weight).  y : [M, N] dtype.
 *   fp32 accumulation.  bf16 with N % 32 == 0 and K % 64 == 0 runs on the MFMA path.
 */
int linear_bt(const void* x, const void* w, void* y, int M, int N, int K, int dtype, void* stream);

/*
 * linear_bt_multi - several linear maps of one input in one product: the weights stacked
 * row-wise in w, each map's result written to its own buffer (the projections that read the
 * same input, "Hybrid attention (§2.3)": kv_proj, the compressor gate, the indexer's key
 * content, gate and head weights, the query's first factor).
 *
 *   x : [M, K] dtype.  w : [sum(widths), K] dtype, map s in rows sum(widths[0..s-1]) onward.
 *   outs[s] : [M, widths[s]] row-major, fp32 when out_f32[s] = 1 else dtype (bf16 inputs may
 *   give fp32 outputs; fp32 inputs give fp32 only).  1 <= n_out <= 8.  fp32 accumulation.
 *   Outputs are overwritten; no buffer may overlap another or x.  bf16 with K % 64 == 0 and
 *   every width a multiple of 32 runs on the MFMA path, other shapes on a plain kernel.
 *   Errors: DSV4_ERR_INVALID for a bad count, width, flag or pointer.
 */
int linear_bt_multi(const void* x, const void* w, int M, int K, int n_out, void* const* outs,
                    const int* widths, const int* out_f32, int dtype, void* stream);

/*
 * input_projections - the projections that make one attention layer's per-token inputs from
 * its hidden state ("Hybrid attention (§2.3)": kv_proj's single K=V head, CSA's compressor
 * gate and the Lightning Indexer of eqs. 13-17; "DeepseekV4Config": q_lora_rank,
 * index_n_heads, index_head_dim; attention_bias False).  Reading: plain linear maps, no bias,
 * no norm between the query factors; the query latent c_q = x . W_qa^T feeds the attention
 * query q and the indexer query q_idx, every other output reads x.
 *
 *   kind  : 0 sliding (c_q, q, kv), 2 HCA (adds gate), 1 CSA (adds gate, q_idx, k_idx, g_idx,
 *           w_idx).  Outputs a layer type does not have are ignored (may be NULL).
 *   x     : [T, hidden] dtype.
 *   w_x   : rows [W_qa (q_rank) | W_kv (D) | W_gate (D) | W_kI (cI) | W_gI (cI) | W_wI (nI)]
 *           of length hidden, the layer's subset in this order, dtype.
 *   w_lat : rows [W_qb (H * D) | W_qI (nI * cI)] of length q_rank (W_qI for CSA only), dtype.
 *   c_q [T, q_rank], q [T, H, D], kv, gate [T, D], q_idx [T, nI, cI], k_idx, g_idx [T, cI]:
 *           dtype (c_q is written first and read back, so it is stored in dtype).
 *   w_idx [T, nI] fp32.  Two launches on `stream`; fp32 accumulation.
 *   Errors: DSV4_ERR_INVALID for a bad kind, size or missing output.
 */
int input_projections(int kind, const void* x, const void* w_x, const void* w_lat, void* c_q, void* q,
                      void* kv, void* gate, void* q_idx, void* k_idx, void* g_idx, float* w_idx, int T,
                      int hidden, int q_rank, int H, int D, int nI, int cI, int dtype, void* stream);

/*
 * attention_mask_dump - render one layer's attention visibility for auditing ("Attention mask
 * layout": the sliding / CSA / HCA mask diagrams of the 16-token example and the audit script
 * described with them, which draws the masks as SVG, prints a terminal grid and dumps the
 * indexer's per-query selections so that warm-up sentinels and picks can be checked).
 * Host code only: no device memory is touched.
 *
 * Rows are queries t = 0 .. S-1 at sequence indices q_pos0 + t.  Columns are the key
 * positions 0 .. q_pos0 + S - 1, then one column per compressed entry C_0 .. C_{n_entries-1}
 * (the entry-visibility view, not gather slots).  Key j is visible to the query at p when
 * max(0, p - window + 1) <= j <= p.  Entry w can be visible once w < min((p + 1) / m,
 * n_entries); HCA (kind 2) marks every such entry, CSA (kind 1) marks the entries its index
 * list selects, shows the other candidates as visible-but-not-selected, and flags a listed
 * entry that is not visible.  A sliding layer (kind 0) has no entry columns.
 *
 *   kind : 0 sliding, 1 CSA, 2 HCA.  m : compress rate (kind 1, 2).
 *   topk_idx : host int32 [S][k] (kind 1; the lists csa_index_topk wrote, -1 = empty slot).
 *   format : 0 plain text grid, 1 the same with ANSI colours, 2 SVG, 3 per-query index lists
 *            with the count of empty slots.
 *   buf, buf_bytes : caller-owned output buffer; *needed receives the bytes the output takes
 *            (including the terminating NUL).  With buf NULL or too small nothing is written
 *            and DSV4_ERR_WORKSPACE is returned, so a first call with buf = NULL sizes it.
 *   At most 2^24 cells (S x columns): DSV4_ERR_UNSUPPORTED beyond.
 */
int attention_mask_dump(int kind, int S, int window, int m, const int* topk_idx, int k,
                        int n_entries, long long q_pos0, int format, char* buf, size_t buf_bytes,
                        size_t* needed);

#ifdef __cplusplus
}
#endif

#endif /* DSV4ATTN_H */
