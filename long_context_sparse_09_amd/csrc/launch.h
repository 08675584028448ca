// Internal kernel launchers of the dsv4attn library (host side, called after validation).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include <string>

namespace dsv4 {

// Records msg as the calling thread's last error detail and returns status.
int report_error(int status, const char* msg);

// x_prev / gate_prev: NULL, or the second projection the earlier half of each overlapping
// window reads (overlap only).
hipError_t launch_compress(const void* x, const void* gate, const void* x_prev, const void* gate_prev,
                           const float* bias, void* pool, int B, int S, int C, int m, int overlap, int e0,
                           int e1, int N_cap, int r, double theta, long long off, int dtype, hipStream_t st);

// Decode-time compressor state: new token rows, rings of the last span tokens, pool.  The
// xp_* / gp_* members are the second projection (NULL: one projection for both halves).
struct CacheUpdate {
  const void* x_new;
  const void* g_new;
  void* x_ring;
  void* g_ring;
  const void* xp_new;
  const void* gp_new;
  void* xp_ring;
  void* gp_ring;
  const float* bias;
  void* pool;
  const int* lengths;
};
hipError_t launch_cache_update(const CacheUpdate& u, int B, int C, int m, int overlap, int N_cap, int r,
                               double theta, long long off, int emit, int dtype, hipStream_t st);
// n (1 or 2) compressors that share lengths, m, overlap and N_cap, in one launch; compressor i
// has width Cs[i] and rotary width rs[i].
hipError_t launch_cache_update(const CacheUpdate* us, const int* Cs, const int* rs, int n, int B, int m, int overlap,
                               int N_cap, double theta, long long off, int emit, int dtype, hipStream_t st);

hipError_t launch_swa(const void* kv_raw, void* kv_win, const int* kv_pos0, const int* new_pos0,
                      int B, int S_new, int S_cap, int D, int r, double theta, long long off,
                      int dtype, hipStream_t st);

// Scores of every visible (query, entry) pair into scores[B*T][N_cap] (fp32).
hipError_t launch_index_scores(const void* q_idx, const float* w_idx, const void* k_pool,
                               const int* q_pos0, const int* n_pool, float* scores, int B, int T,
                               int nI, int cI, int N_cap, int m, int dtype, hipStream_t st);

// Top-k selection from scores[B*T][N_cap].
hipError_t launch_topk(const float* scores, const int* q_pos0, const int* n_pool, int* topk_idx,
                       float* topk_score, int B, int T, int N_cap, int m, int k, hipStream_t st);

struct AttendArgs {
  const void* q;
  const void* kv_win;
  const int* kv_pos0;
  int S_kv;
  const void* pool;
  int N_cap;
  const int* topk_idx;  // CSA: [B,T,k]; HCA: NULL
  int k;
  const int* n_pool;  // HCA: [B] or NULL
  int m_hca;
  const float* sink;
  const int* q_pos0;
  void* out;
  int B, T, H, D, window, r;
  double theta;
  long long pos_off;
  float scale;
  int dtype;
  bool csa;
  double inv_freq[128];  // theta^(-2i/r), i < r/2, formed on the host in double precision
  // Split mode (few queries): each query's keys are cut into n_split ranges scored by separate
  // workgroups; part holds their fp32 partial outputs [items][H][D] then (max, sum) pairs
  // [items][H][2], merged by a second kernel.  n_split = 1: part unused.
  int n_split;
  float* part;
  // hca_attend_pairs: the query-pair kernel (two consecutive queries share each key tile)
  bool pairs;
};

// Key ranges per query the split mode uses for n_q queries on this device (1: no split), and
// the workspace it needs.
int attend_split_count(int n_q);
size_t attend_split_bytes(int n_q);

hipError_t launch_attend(const AttendArgs& a, hipStream_t st);

// Dense-range attention over query pairs (HCA and sliding layers): whether the kernel covers a
// shape, and the launch.
bool attend_dense_fits(const AttendArgs& a);
hipError_t launch_attend_dense(const AttendArgs& a, hipStream_t st);

// Whether the MFMA fast paths cover a shape (otherwise the generic kernels run).
bool index_scores_fast(int nI, int cI, int dtype);
bool attend_fast(int H, int D, int r, int dtype);
bool attend_uses_fast(const AttendArgs& a);
// Keys one query may see at most (sizes the generic attention kernel's LDS).
int attend_generic_max_keys();

// C[M,N] = A[M,K] . B[N,K]^T per batch entry g (A, B, C offset by g * sA, sB, sC elements).
hipError_t launch_gemm_bt(const void* A, const void* B, void* C, int M, int N, int K, long long lda,
                          long long ldb, long long ldc, int batch, long long sA, long long sB, long long sC,
                          int dtype, hipStream_t st);

// The columns of C split into consecutive segments, each stored in its own buffer: segment s
// holds columns begin[s] .. begin[s+1]-1 as a row-major [M, begin[s+1]-begin[s]] array with
// rows of stride ld[s] elements, batch entry g at ptr[s] + g * stride[s] elements, in fp32
// (f32[s] = 1) or bf16 (0).  begin[0] = 0 and begin[n_seg] = N.
constexpr int kGemmMaxSeg = 8;
struct GemmOut {
  int n_seg;
  int begin[kGemmMaxSeg + 1];
  int f32[kGemmMaxSeg];
  long long ld[kGemmMaxSeg];
  long long stride[kGemmMaxSeg];
  void* ptr[kGemmMaxSeg];
};
hipError_t launch_gemm_bt_seg(const void* A, const void* B, const GemmOut& out, int M, int K, long long lda,
                              long long ldb, int batch, long long sA, long long sB, int dtype, hipStream_t st);
bool gemm_fast(const GemmOut& out, int K, long long lda, long long ldb, int dtype);

// Visibility rendering of one layer (host only).  kind 0 sliding, 1 CSA, 2 HCA; format 0 text,
// 1 ANSI text, 2 SVG, 3 per-query index lists.  topk_idx: host [S][k] (CSA).
struct MaskDumpArgs {
  int kind, S, window, m, k, n_entries, format;
  long long q_pos0;
  const int* topk_idx;
};
std::string render_mask(const MaskDumpArgs& a);

}  // namespace dsv4
