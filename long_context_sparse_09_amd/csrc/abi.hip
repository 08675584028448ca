// Host side of the dsv4attn C ABI: argument validation, kernel dispatch, status reporting.
// Declarations and argument meaning: include/dsv4attn.h.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/dsv4attn.h"
#include "common.h"
#include "launch.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return DSV4_OK;
}

}  // namespace

// Status reporting for entry points defined in other source files of the library.
int dsv4::report_error(int status, const char* msg) { return fail(status, "%s", msg); }

namespace {

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DSV4_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dtype_ok(int dtype) { return dtype == DSV4_FP32 || dtype == DSV4_BF16; }

#define REQUIRE(cond, ...)                                  \
  do {                                                      \
    if (!(cond)) return fail(DSV4_ERR_INVALID, __VA_ARGS__); \
  } while (0)

int check_rope(int rope_dim, int C, double theta) {
  REQUIRE(rope_dim >= 0 && rope_dim % 2 == 0 && rope_dim <= C, "rope_dim %d must be even and in [0, %d]", rope_dim, C);
  if (rope_dim > dsv4::kMaxRope) return fail(DSV4_ERR_UNSUPPORTED, "rope_dim %d above %d", rope_dim, dsv4::kMaxRope);
  REQUIRE(rope_dim == 0 || theta > 0.0, "rope_theta must be positive");
  return DSV4_OK;
}

}  // namespace

extern "C" {

int dsv4_abi_version(void) { return DSV4_ABI_VERSION; }

const char* dsv4_status_string(int status) {
  switch (status) {
    case DSV4_OK: return "ok";
    case DSV4_ERR_INVALID: return "invalid argument";
    case DSV4_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case DSV4_ERR_LAUNCH: return "kernel launch failed";
    case DSV4_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

const char* dsv4_last_error(void) { return g_last_error; }

}  // extern "C"

namespace {

int compress_common(const void* x, const void* gate, const void* x_prev, const void* gate_prev,
                    const float* bias, void* pool, int B, int S, int C, int m, int overlap, int entry_begin,
                    int entry_end, int N_cap, int rope_dim, double rope_theta, long long rope_pos_offset,
                    int dtype, void* stream, const char* name) {
  REQUIRE(dtype_ok(dtype), "dtype %d", dtype);
  REQUIRE(B >= 0 && S >= 0 && N_cap >= 0, "negative size");
  REQUIRE(m >= 1, "m must be >= 1");
  REQUIRE(overlap == 0 || overlap == 1, "overlap must be 0 or 1");
  REQUIRE(C >= 2 && C % 2 == 0, "C must be even and >= 2");
  if (!(C % 8 == 0 ? C <= 2048 : C <= 512))
    return fail(DSV4_ERR_UNSUPPORTED, "C=%d: need C <= 2048 (multiple of 8) or <= 512", C);
  REQUIRE(0 <= entry_begin && entry_begin <= entry_end && entry_end <= N_cap,
          "entries [%d,%d) outside [0,N_cap=%d]", entry_begin, entry_end, N_cap);
  REQUIRE(static_cast<long long>(entry_end) * m <= S, "entry %d's window is not closed by S=%d", entry_end - 1, S);
  if (int rc = check_rope(rope_dim, C, rope_theta)) return rc;
  if (B == 0 || entry_begin == entry_end) return ok();
  REQUIRE(x && gate && pool, "null x/gate/pool");
  REQUIRE(aligned16(x) && aligned16(gate) && aligned16(pool) && (!bias || aligned16(bias)) &&
              (!x_prev || aligned16(x_prev)) && (!gate_prev || aligned16(gate_prev)),
          "pointers must be 16-byte aligned");
  return launched(dsv4::launch_compress(x, gate, x_prev, gate_prev, bias, pool, B, S, C, m, overlap, entry_begin,
                                        entry_end, N_cap, rope_dim, rope_theta, rope_pos_offset, dtype,
                                        static_cast<hipStream_t>(stream)),
                  name);
}

// Argument checks of one compressor cache update; DSV4_OK (0) when it may launch.  *empty is
// set when there is nothing to do (B == 0).
int cache_update_check(const dsv4::CacheUpdate& u, int B, int C, int m, int overlap, int N_cap, int rope_dim,
                       double rope_theta, int emit, int dtype, bool* empty) {
  *empty = false;
  REQUIRE(dtype_ok(dtype), "dtype %d", dtype);
  REQUIRE(B >= 0 && N_cap >= 0, "negative size");
  REQUIRE(m >= 1, "m must be >= 1");
  REQUIRE(overlap == 0 || overlap == 1, "overlap must be 0 or 1");
  REQUIRE(C >= 2 && C % 2 == 0, "C must be even and >= 2");
  if (!(C % 8 == 0 ? C <= 2048 : C <= 512))
    return fail(DSV4_ERR_UNSUPPORTED, "C=%d: need C <= 2048 (multiple of 8) or <= 512", C);
  if ((overlap ? 2 * m : m) > 4096) return fail(DSV4_ERR_UNSUPPORTED, "window span above 4096");
  if (int rc = check_rope(rope_dim, C, rope_theta)) return rc;
  if (B == 0) {
    *empty = true;
    return ok();
  }
  REQUIRE(u.x_new && u.g_new && u.x_ring && u.g_ring && u.lengths, "null required pointer");
  REQUIRE(!emit || u.pool, "pool required when emitting entries");
  for (const void* p : {u.x_new, u.g_new, static_cast<const void*>(u.x_ring), static_cast<const void*>(u.g_ring),
                        u.xp_new, u.gp_new, static_cast<const void*>(u.xp_ring), static_cast<const void*>(u.gp_ring),
                        static_cast<const void*>(u.pool), static_cast<const void*>(u.bias)})
    REQUIRE(!p || aligned16(p), "pointers must be 16-byte aligned");
  return ok();
}

int cache_update_common(const dsv4::CacheUpdate& u, int B, int C, int m, int overlap, int N_cap, int rope_dim,
                        double rope_theta, long long rope_pos_offset, int emit, int dtype, void* stream,
                        const char* name) {
  bool empty = false;
  if (int rc = cache_update_check(u, B, C, m, overlap, N_cap, rope_dim, rope_theta, emit, dtype, &empty)) return rc;
  if (empty) return ok();
  return launched(dsv4::launch_cache_update(u, B, C, m, overlap, N_cap, rope_dim, rope_theta, rope_pos_offset, emit,
                                            dtype, static_cast<hipStream_t>(stream)),
                  name);
}

}  // namespace

extern "C" {

int csa_compress(const void* x, const void* gate, const float* bias, void* pool, int B, int S,
                 int C, int m, int overlap, int entry_begin, int entry_end, int N_cap,
                 int rope_dim, double rope_theta, long long rope_pos_offset, int dtype,
                 void* stream) {
  return compress_common(x, gate, nullptr, nullptr, bias, pool, B, S, C, m, overlap, entry_begin, entry_end,
                         N_cap, rope_dim, rope_theta, rope_pos_offset, dtype, stream, "csa_compress");
}

int csa_compress_split(const void* x, const void* gate, const void* x_prev, const void* gate_prev,
                       const float* bias, void* pool, int B, int S, int C, int m, int entry_begin,
                       int entry_end, int N_cap, int rope_dim, double rope_theta, long long rope_pos_offset,
                       int dtype, void* stream) {
  REQUIRE((x_prev == nullptr) == (gate_prev == nullptr), "x_prev and gate_prev go together");
  return compress_common(x, gate, x_prev, gate_prev, bias, pool, B, S, C, m, 1, entry_begin, entry_end, N_cap,
                         rope_dim, rope_theta, rope_pos_offset, dtype, stream, "csa_compress_split");
}

int compressor_cache_update(const void* x_new, const void* gate_new, void* x_ring,
                            void* gate_ring, const float* bias, void* pool, const int* lengths,
                            int B, int C, int m, int overlap, int N_cap, int rope_dim,
                            double rope_theta, long long rope_pos_offset, int emit, int dtype,
                            void* stream) {
  const dsv4::CacheUpdate u{x_new, gate_new, x_ring, gate_ring, nullptr, nullptr, nullptr, nullptr, bias, pool,
                            lengths};
  return cache_update_common(u, B, C, m, overlap, N_cap, rope_dim, rope_theta, rope_pos_offset, emit, dtype,
                             stream, "compressor_cache_update");
}

int compressor_cache_update_pair(const void* x_new, const void* gate_new, void* x_ring, void* gate_ring,
                                 const float* bias, void* pool, int C, int rope_dim, const void* x2_new,
                                 const void* gate2_new, void* x2_ring, void* gate2_ring, const float* bias2,
                                 void* pool2, int C2, int rope_dim2, const int* lengths, int B, int m, int overlap,
                                 int N_cap, double rope_theta, long long rope_pos_offset, int emit, int dtype,
                                 void* stream) {
  const dsv4::CacheUpdate u[2] = {
      {x_new, gate_new, x_ring, gate_ring, nullptr, nullptr, nullptr, nullptr, bias, pool, lengths},
      {x2_new, gate2_new, x2_ring, gate2_ring, nullptr, nullptr, nullptr, nullptr, bias2, pool2, lengths}};
  const int Cs[2] = {C, C2}, rs[2] = {rope_dim, rope_dim2};
  bool empty = false;
  for (int i = 0; i < 2; ++i)
    if (int rc = cache_update_check(u[i], B, Cs[i], m, overlap, N_cap, rs[i], rope_theta, emit, dtype, &empty))
      return rc;
  if (empty) return ok();
  return launched(dsv4::launch_cache_update(u, Cs, rs, 2, B, m, overlap, N_cap, rope_theta, rope_pos_offset, emit,
                                            dtype, static_cast<hipStream_t>(stream)),
                  "compressor_cache_update_pair");
}

int compressor_cache_update_split(const void* x_new, const void* gate_new, const void* x_prev_new,
                                  const void* gate_prev_new, void* x_ring, void* gate_ring, void* x_prev_ring,
                                  void* gate_prev_ring, const float* bias, void* pool, const int* lengths, int B,
                                  int C, int m, int N_cap, int rope_dim, double rope_theta,
                                  long long rope_pos_offset, int emit, int dtype, void* stream) {
  REQUIRE(x_prev_new && gate_prev_new && x_prev_ring && gate_prev_ring, "null second-projection pointer");
  const dsv4::CacheUpdate u{x_new, gate_new, x_ring, gate_ring, x_prev_new, gate_prev_new, x_prev_ring,
                            gate_prev_ring, bias, pool, lengths};
  return cache_update_common(u, B, C, m, 1, N_cap, rope_dim, rope_theta, rope_pos_offset, emit, dtype, stream,
                             "compressor_cache_update_split");
}

int linear_bt(const void* x, const void* w, void* y, int M, int N, int K, int dtype, void* stream) {
  REQUIRE(dtype_ok(dtype), "dtype %d", dtype);
  REQUIRE(M >= 0 && N >= 1 && K >= 1, "M >= 0, N >= 1, K >= 1 required");
  if (M == 0) return ok();
  REQUIRE(x && w && y, "null x/w/y");
  REQUIRE(aligned16(x) && aligned16(w) && aligned16(y), "pointers must be 16-byte aligned");
  return launched(dsv4::launch_gemm_bt(x, w, y, M, N, K, K, K, N, 1, 0, 0, 0, dtype,
                                       static_cast<hipStream_t>(stream)),
                  "linear_bt");
}

int grouped_out_proj(const void* attn, const void* w_a, const void* w_b, void* mid, void* out, int T,
                     int H, int D, int groups, int rank, int hidden, int dtype, void* stream) {
  REQUIRE(dtype_ok(dtype), "dtype %d", dtype);
  REQUIRE(T >= 0 && H >= 1 && D >= 1 && rank >= 1 && hidden >= 1, "sizes must be positive");
  REQUIRE(groups >= 1 && H % groups == 0, "groups %d must divide H=%d", groups, H);
  if (static_cast<long long>(T) * H * D * 2 >= (1LL << 31) ||
      static_cast<long long>(T) * groups * rank * 2 >= (1LL << 31) ||
      static_cast<long long>(T) * hidden * 2 >= (1LL << 31))
    return fail(DSV4_ERR_UNSUPPORTED, "a [T, .] operand of 2 GiB or more: split T");
  if (T == 0) return ok();
  REQUIRE(attn && w_a && w_b && mid && out, "null attn/w_a/w_b/mid/out");
  REQUIRE(aligned16(attn) && aligned16(w_a) && aligned16(w_b) && aligned16(mid) && aligned16(out),
          "pointers must be 16-byte aligned");
  const long long kg = static_cast<long long>(H / groups) * D;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = dsv4::launch_gemm_bt(attn, w_a, mid, T, rank, static_cast<int>(kg), static_cast<long long>(H) * D,
                                      kg, static_cast<long long>(groups) * rank, groups, kg, rank * kg, rank,
                                      dtype, st);
  if (e != hipSuccess) return launched(e, "grouped_out_proj (o_a)");
  return launched(dsv4::launch_gemm_bt(mid, w_b, out, T, hidden, groups * rank, static_cast<long long>(groups) * rank,
                                       static_cast<long long>(groups) * rank, hidden, 1, 0, 0, 0, dtype, st),
                  "grouped_out_proj (o_b)");
}

int linear_bt_multi(const void* x, const void* w, int M, int K, int n_out, void* const* outs, const int* widths,
                    const int* out_f32, int dtype, void* stream) {
  REQUIRE(dtype_ok(dtype), "dtype %d", dtype);
  REQUIRE(M >= 0 && K >= 1, "M >= 0 and K >= 1 required");
  REQUIRE(n_out >= 1 && n_out <= dsv4::kGemmMaxSeg, "n_out %d outside [1, %d]", n_out, dsv4::kGemmMaxSeg);
  REQUIRE(outs && widths && out_f32, "null outs/widths/out_f32");
  dsv4::GemmOut o{};
  o.n_seg = n_out;
  long long N = 0;
  for (int s = 0; s < n_out; ++s) {
    REQUIRE(widths[s] >= 1, "widths[%d] = %d must be >= 1", s, widths[s]);
    REQUIRE(out_f32[s] == 0 || out_f32[s] == 1, "out_f32[%d] must be 0 or 1", s);
    REQUIRE(dtype == DSV4_BF16 || out_f32[s] == 1, "fp32 inputs give fp32 outputs only");
    o.begin[s] = static_cast<int>(N);
    N += widths[s];
    o.f32[s] = out_f32[s];
    o.ld[s] = widths[s];
    o.ptr[s] = outs[s];
  }
  REQUIRE(N < (1LL << 30), "total width %lld too large", N);
  o.begin[n_out] = static_cast<int>(N);
  if (M == 0) return ok();
  REQUIRE(x && w, "null x/w");
  REQUIRE(aligned16(x) && aligned16(w), "pointers must be 16-byte aligned");
  for (int s = 0; s < n_out; ++s) REQUIRE(outs[s] && aligned16(outs[s]), "outs[%d] null or not 16-byte aligned", s);
  return launched(dsv4::launch_gemm_bt_seg(x, w, o, M, K, K, K, 1, 0, 0, dtype, static_cast<hipStream_t>(stream)),
                  "linear_bt_multi");
}

int input_projections(int kind, const void* x, const void* w_x, const void* w_lat, void* c_q, void* q, void* kv,
                      void* gate, void* q_idx, void* k_idx, void* g_idx, float* w_idx, int T, int hidden,
                      int q_rank, int H, int D, int nI, int cI, int dtype, void* stream) {
  REQUIRE(kind >= 0 && kind <= 2, "kind %d: 0 sliding, 1 CSA, 2 HCA", kind);
  REQUIRE(dtype_ok(dtype), "dtype %d", dtype);
  REQUIRE(T >= 0 && hidden >= 1 && q_rank >= 1 && H >= 1 && D >= 1, "sizes must be positive");
  REQUIRE(kind != 1 || (nI >= 1 && cI >= 1), "CSA needs nI, cI >= 1");
  REQUIRE(static_cast<long long>(H) * D < (1LL << 28) && static_cast<long long>(nI) * cI < (1LL << 28),
          "query width too large");
  // stage 1 reads x: [c_q | kv | gate | k_idx | g_idx | w_idx] (the layer's subset, in this order)
  void* o1[6] = {c_q, kv, gate, k_idx, g_idx, w_idx};
  const int wd1[6] = {q_rank, D, D, cI, cI, nI};
  const int f1[6] = {dtype == DSV4_FP32, dtype == DSV4_FP32, dtype == DSV4_FP32, dtype == DSV4_FP32,
                     dtype == DSV4_FP32, 1};
  const int n1 = kind == 0 ? 2 : kind == 2 ? 3 : 6;
  // stage 2 reads c_q: [q | q_idx]
  void* o2[2] = {q, q_idx};
  const int wd2[2] = {H * D, kind == 1 ? nI * cI : 0};
  const int f2[2] = {dtype == DSV4_FP32, dtype == DSV4_FP32};
  const int n2 = kind == 1 ? 2 : 1;
  if (T == 0) return ok();
  REQUIRE(x && w_x && w_lat, "null x/w_x/w_lat");
  for (int s = 0; s < n1; ++s) REQUIRE(o1[s], "null output %d of the hidden-state projections", s);
  for (int s = 0; s < n2; ++s) REQUIRE(o2[s], "null output %d of the latent projections", s);
  int rc = linear_bt_multi(x, w_x, T, hidden, n1, o1, wd1, f1, dtype, stream);
  if (rc != DSV4_OK) return rc;
  return linear_bt_multi(c_q, w_lat, T, q_rank, n2, o2, wd2, f2, dtype, stream);
}

int attention_mask_dump(int kind, int S, int window, int m, const int* topk_idx, int k,
                        int n_entries, long long q_pos0, int format, char* buf, size_t buf_bytes,
                        size_t* needed) {
  REQUIRE(kind >= 0 && kind <= 2, "kind %d: 0 sliding, 1 CSA, 2 HCA", kind);
  REQUIRE(format >= 0 && format <= 3, "format %d: 0 text, 1 ANSI, 2 SVG, 3 index lists", format);
  REQUIRE(S >= 0 && q_pos0 >= 0 && window >= 1, "S, q_pos0 must be >= 0 and window >= 1");
  REQUIRE(kind == 0 || (m >= 1 && n_entries >= 0), "m must be >= 1 and n_entries >= 0");
  REQUIRE(kind != 1 || (k >= 1 && (S == 0 || topk_idx)), "CSA needs the index lists (k >= 1)");
  REQUIRE(needed != nullptr, "needed must not be NULL");
  const long long width = q_pos0 + S + (kind == 0 ? 0 : n_entries);
  if (static_cast<long long>(S) * width > (1LL << 24))
    return fail(DSV4_ERR_UNSUPPORTED, "%lld cells: at most 2^24", static_cast<long long>(S) * width);
  dsv4::MaskDumpArgs a{kind, S, window, m, kind == 1 ? k : 0, kind == 0 ? 0 : n_entries, format, q_pos0,
                       topk_idx};
  const std::string out = dsv4::render_mask(a);
  *needed = out.size() + 1;
  if (buf == nullptr || buf_bytes < out.size() + 1)
    return fail(DSV4_ERR_WORKSPACE, "output needs %zu bytes", out.size() + 1);
  memcpy(buf, out.c_str(), out.size() + 1);
  return ok();
}

size_t csa_index_topk_workspace_size(int B, int T, int N_cap, int k) {
  (void)k;
  if (B <= 0 || T <= 0 || N_cap <= 0) return 0;
  return static_cast<size_t>(B) * T * N_cap * sizeof(float);
}

int csa_index_topk(const void* q_idx, const float* w_idx, const void* k_pool, const int* q_pos0,
                   const int* n_pool, int* topk_idx, float* topk_score, int B, int T, int nI,
                   int cI, int N_cap, int m, int k, void* workspace, size_t workspace_bytes,
                   int dtype, void* stream) {
  REQUIRE(dtype_ok(dtype), "dtype %d", dtype);
  REQUIRE(B >= 0 && T >= 0, "negative size");
  REQUIRE(nI >= 1 && cI >= 1, "nI, cI must be >= 1");
  REQUIRE(m >= 1, "m must be >= 1");
  REQUIRE(N_cap >= 1 && N_cap <= (1 << 20), "N_cap %d outside [1, 2^20]", N_cap);
  REQUIRE(k >= 1 && k <= N_cap, "k %d outside [1, N_cap=%d]", k, N_cap);
  if (k > 4096) return fail(DSV4_ERR_UNSUPPORTED, "k %d above 4096", k);
  if (!dsv4::index_scores_fast(nI, cI, dtype) && nI * cI + nI > 16384)
    return fail(DSV4_ERR_UNSUPPORTED, "nI*cI=%d too large for the generic indexer", nI * cI);
  if (B == 0 || T == 0) return ok();
  REQUIRE(q_idx && w_idx && k_pool && q_pos0 && n_pool && topk_idx, "null required pointer");
  REQUIRE(aligned16(q_idx) && aligned16(k_pool) && aligned16(w_idx), "pointers must be 16-byte aligned");
  const size_t need = csa_index_topk_workspace_size(B, T, N_cap, k);
  if (!workspace || workspace_bytes < need)
    return fail(DSV4_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  float* scores = static_cast<float*>(workspace);
  hipError_t e = dsv4::launch_index_scores(q_idx, w_idx, k_pool, q_pos0, n_pool, scores, B, T, nI,
                                           cI, N_cap, m, dtype, st);
  if (e != hipSuccess) return launched(e, "csa_index_topk (scores)");
  return launched(dsv4::launch_topk(scores, q_pos0, n_pool, topk_idx, topk_score, B, T, N_cap, m,
                                    k, st),
                  "csa_index_topk (select)");
}

int swa_concat(const void* kv_raw, void* kv_win, const int* kv_pos0, const int* new_pos0, int B,
               int S_new, int S_cap, int D, int rope_dim, double rope_theta,
               long long rope_pos_offset, int dtype, void* stream) {
  REQUIRE(dtype_ok(dtype), "dtype %d", dtype);
  REQUIRE(B >= 0 && S_new >= 0 && S_cap >= 0, "negative size");
  REQUIRE(D >= 2 && D % 2 == 0, "D must be even and >= 2");
  if (int rc = check_rope(rope_dim, D, rope_theta)) return rc;
  if (B == 0 || S_new == 0 || S_cap == 0) return ok();
  if (static_cast<long long>(B) * S_new * D >= (1LL << 32))
    return fail(DSV4_ERR_UNSUPPORTED, "B*S_new*D = %lld elements, at most 2^32 - 1",
                static_cast<long long>(B) * S_new * D);
  REQUIRE(kv_raw && kv_win && kv_pos0 && new_pos0, "null required pointer");
  REQUIRE(aligned16(kv_raw) && aligned16(kv_win), "pointers must be 16-byte aligned");
  return launched(dsv4::launch_swa(kv_raw, kv_win, kv_pos0, new_pos0, B, S_new, S_cap, D, rope_dim,
                                   rope_theta, rope_pos_offset, dtype,
                                   static_cast<hipStream_t>(stream)),
                  "swa_concat");
}

static int attend_common(dsv4::AttendArgs& a, void* workspace, size_t workspace_bytes,
                         void* stream, const char* name) {
  REQUIRE(dtype_ok(a.dtype), "dtype %d", a.dtype);
  REQUIRE(a.B >= 0 && a.T >= 0 && a.S_kv >= 0 && a.N_cap >= 0, "negative size");
  REQUIRE(a.H >= 1 && a.D >= 2 && a.D % 2 == 0, "H >= 1 and even D >= 2 required");
  REQUIRE(a.window >= 1, "window must be >= 1");
  if (int rc = check_rope(a.r, a.D, a.theta)) return rc;
  if (a.scale <= 0.f) a.scale = 1.0f / sqrtf(static_cast<float>(a.D));
  for (int i = 0; i < a.r / 2; ++i) a.inv_freq[i] = pow(a.theta, -2.0 * i / a.r);
  if (a.B == 0 || a.T == 0) return ok();
  REQUIRE(a.q && a.kv_win && a.kv_pos0 && a.sink && a.q_pos0 && a.out, "null required pointer");
  REQUIRE(a.N_cap == 0 || a.pool, "pool required when N_cap > 0");
  REQUIRE(aligned16(a.q) && aligned16(a.kv_win) && aligned16(a.out) && (!a.pool || aligned16(a.pool)),
          "pointers must be 16-byte aligned");
  a.n_split = 1;
  a.part = nullptr;
  if (workspace != nullptr) {
    REQUIRE(aligned16(workspace), "workspace must be 16-byte aligned");
    const size_t need = dsv4::attend_split_bytes(a.B * a.T);
    if (workspace_bytes < need)
      return fail(DSV4_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
    if (need > 0 && dsv4::attend_uses_fast(a)) {
      a.n_split = dsv4::attend_split_count(a.B * a.T);
      a.part = static_cast<float*>(workspace);
    }
  }
  if (!dsv4::attend_uses_fast(a)) {
    if (a.D > 4096) return fail(DSV4_ERR_UNSUPPORTED, "D=%d above 4096 for the generic kernel", a.D);
    const long long max_keys = static_cast<long long>(a.window) + (a.csa ? a.k : a.N_cap);
    if (max_keys > dsv4::attend_generic_max_keys())
      return fail(DSV4_ERR_UNSUPPORTED, "%lld keys per query exceed the generic kernel's %d", max_keys,
                  dsv4::attend_generic_max_keys());
  }
  return launched(dsv4::launch_attend(a, static_cast<hipStream_t>(stream)), name);
}

size_t attend_workspace_size(int B, int T, int H, int D) {
  if (B <= 0 || T <= 0 || !dsv4::attend_fast(H, D, 0, 1)) return 0;
  return dsv4::attend_split_bytes(B * T);
}

int csa_attend(const void* q, const void* kv_win, const int* kv_pos0, int S_kv, const void* pool,
               int N_cap, const int* topk_idx, int k, const float* sink, const int* q_pos0,
               void* out, int B, int T, int H, int D, int window, int rope_dim,
               double rope_theta, long long rope_pos_offset, float scale, void* workspace,
               size_t workspace_bytes, int dtype, void* stream) {
  REQUIRE(k >= 1, "k must be >= 1");
  if (k > 4096) return fail(DSV4_ERR_UNSUPPORTED, "k %d above 4096", k);
  REQUIRE(B == 0 || T == 0 || topk_idx, "null topk_idx");
  dsv4::AttendArgs a{q, kv_win, kv_pos0, S_kv, pool, N_cap, topk_idx, k, nullptr, 1, sink, q_pos0,
                     out, B, T, H, D, window, rope_dim, rope_theta, rope_pos_offset, scale, dtype, true,
                     {}};
  return attend_common(a, workspace, workspace_bytes, stream, "csa_attend");
}

int hca_attend(const void* q, const void* kv_win, const int* kv_pos0, int S_kv, const void* pool,
               int N_cap, const int* n_pool, int m_hca, const float* sink, const int* q_pos0,
               void* out, int B, int T, int H, int D, int window, int rope_dim,
               double rope_theta, long long rope_pos_offset, float scale, void* workspace,
               size_t workspace_bytes, int dtype, void* stream) {
  REQUIRE(m_hca >= 1, "m_hca must be >= 1");
  dsv4::AttendArgs a{q, kv_win, kv_pos0, S_kv, pool, N_cap, nullptr, 0, n_pool, m_hca, sink, q_pos0,
                     out, B, T, H, D, window, rope_dim, rope_theta, rope_pos_offset, scale, dtype, false,
                     {}};
  return attend_common(a, workspace, workspace_bytes, stream, "hca_attend");
}

int hca_attend_pairs(const void* q, const void* kv_win, const int* kv_pos0, int S_kv, const void* pool,
                     int N_cap, const int* n_pool, int m_hca, const float* sink, const int* q_pos0,
                     void* out, int B, int T, int H, int D, int window, int rope_dim,
                     double rope_theta, long long rope_pos_offset, float scale, int dtype,
                     void* stream) {
  REQUIRE(m_hca >= 1, "m_hca must be >= 1");
  dsv4::AttendArgs a{q, kv_win, kv_pos0, S_kv, pool, N_cap, nullptr, 0, n_pool, m_hca, sink, q_pos0,
                     out, B, T, H, D, window, rope_dim, rope_theta, rope_pos_offset, scale, dtype, false,
                     {}};
  if (!dsv4::attend_dense_fits(a))
    return fail(DSV4_ERR_UNSUPPORTED, "hca_attend_pairs covers bf16, H = 64, D = 512, rope_dim 0 or 64 only");
  a.pairs = true;
  return attend_common(a, nullptr, 0, stream, "hca_attend_pairs");
}

}  // extern "C"
