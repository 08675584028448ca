// Generic shared-K=V attention with sink, sliding window and compressed keys (any H, D;
// fp32 or bf16 storage, fp32 arithmetic).  Serves the fp32 dtype and every shape the MFMA
// kernel does not cover.
//
// Source: DeepSeek-V4 model page (Transformers docs), "Hybrid attention (§2.3)": one K=V head
// read as key and value; partial RoPE on the trailing channels; output rope slice rotated at
// position -i (eq. 26); per-head sink (eq. 27); sliding-window K=V branch concatenated before
// the compressed keys.  "Attention mask layout": window cut, CSA -1 sentinel, HCA entry
// visibility w < (t+1)//m.
//
// One block per (query, head).  Phase 1: one thread per key computes its logit.  Phase 2:
// block max / sum including the sink.  Phase 3: one thread per channel pair accumulates the
// weighted keys and applies the counter-rotation.
#include "common.h"
#include "launch.h"

namespace dsv4 {

constexpr int kGenericMaxKeys = 4096;  // 32 KB of logits + key codes in LDS

int attend_generic_max_keys() { return kGenericMaxKeys; }

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = (blockDim.x + 63) >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float o = __shfl_xor(v, off);
    v = is_max ? fmaxf(v, o) : v + o;
  }
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < nw; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  __syncthreads();
  return r;
}

template <typename T>
__global__ void __launch_bounds__(256) attend_generic_kernel(AttendArgs a) {
  extern __shared__ float sm[];
  const int D = a.D, H = a.H;
  float* qs = sm;                          // [D] rotated query
  float* z = qs + D;                       // [max keys] logits, then weights
  int* klist = reinterpret_cast<int*>(z + kGenericMaxKeys);  // key rows: >= 0 pool, < 0 window
  __shared__ float red[16];
  __shared__ double inv_freq[kMaxRope / 2];
  __shared__ int n_keys_sh;

  const int h = blockIdx.x % H;
  const int t = (blockIdx.x / H) % a.T;
  const int b = blockIdx.x / (H * a.T);
  const long long p = static_cast<long long>(a.q_pos0[b]) + t;
  rope_table(inv_freq, a.r, a.theta);

  // key list: window rows first, then compressed entries
  if (threadIdx.x == 0) {
    const long long lo = max(0LL, p - a.window + 1);
    const long long r0 = max(lo - a.kv_pos0[b], 0LL);
    const long long r1 = min(p + 1 - a.kv_pos0[b], static_cast<long long>(a.S_kv));
    int n = 0;
    for (long long rr = r0; rr < r1 && n < kGenericMaxKeys; ++rr) klist[n++] = -1 - static_cast<int>(rr);
    if (a.csa) {
      const int* idx = a.topk_idx + (static_cast<size_t>(b) * a.T + t) * a.k;
      for (int i = 0; i < a.k && n < kGenericMaxKeys; ++i) {
        const int e = idx[i];
        if (e >= 0 && e < a.N_cap) klist[n++] = e;
      }
    } else if (a.N_cap > 0) {
      long long v = (p + 1) / a.m_hca;
      v = min(v, static_cast<long long>(a.n_pool ? a.n_pool[b] : a.N_cap));
      v = min(v, static_cast<long long>(a.N_cap));
      for (int e = 0; e < v && n < kGenericMaxKeys; ++e) klist[n++] = e;
    }
    n_keys_sh = n;
  }
  __syncthreads();
  const int n_keys = n_keys_sh;

  const T* qrow = static_cast<const T*>(a.q) + ((static_cast<size_t>(b) * a.T + t) * H + h) * D;
  const double pos = static_cast<double>(p + a.pos_off);
  for (int c = 2 * threadIdx.x; c < D; c += 2 * blockDim.x) {
    float v[2] = {load1<T>(qrow + c), load1<T>(qrow + c + 1)};
    rope_chunk<2>(v, c, D, a.r, pos, inv_freq);
    qs[c] = v[0];
    qs[c + 1] = v[1];
  }
  __syncthreads();

  const T* win = static_cast<const T*>(a.kv_win) + static_cast<size_t>(b) * a.S_kv * D;
  const T* pool = static_cast<const T*>(a.pool) + static_cast<size_t>(b) * a.N_cap * D;
  auto key_row = [&](int code) -> const T* {
    return code >= 0 ? pool + static_cast<size_t>(code) * D : win + static_cast<size_t>(-1 - code) * D;
  };

  // phase 1: logits
  float lmax = -INFINITY;
  for (int x = threadIdx.x; x < n_keys; x += blockDim.x) {
    const T* kr = key_row(klist[x]);
    float dot = 0.f;
    for (int c = 0; c < D; ++c) dot += qs[c] * load1<T>(kr + c);
    const float zz = dot * a.scale;
    z[x] = zz;
    lmax = fmaxf(lmax, zz);
  }
  const float sink = a.sink[h];
  const float M = fmaxf(block_reduce(lmax, red, true), sink);
  float lsum = 0.f;
  for (int x = threadIdx.x; x < n_keys; x += blockDim.x) {
    const float e = expf(z[x] - M);
    z[x] = e;
    lsum += e;
  }
  const float denom = block_reduce(lsum, red, false) + expf(sink - M);
  __syncthreads();

  // phase 3: weighted keys, counter-rotation, store
  T* orow = static_cast<T*>(a.out) + ((static_cast<size_t>(b) * a.T + t) * H + h) * D;
  for (int c = 2 * threadIdx.x; c < D; c += 2 * blockDim.x) {
    float o0 = 0.f, o1 = 0.f;
    for (int x = 0; x < n_keys; ++x) {
      const T* kr = key_row(klist[x]);
      o0 += z[x] * load1<T>(kr + c);
      o1 += z[x] * load1<T>(kr + c + 1);
    }
    float v[2] = {o0 / denom, o1 / denom};
    rope_chunk<2>(v, c, D, a.r, -pos, inv_freq);
    Chunk<T>::template store<2>(orow + c, v);
  }
}

hipError_t launch_attend_generic(const AttendArgs& a, hipStream_t st) {
  const size_t shmem = static_cast<size_t>(a.D) * sizeof(float) +
                       static_cast<size_t>(kGenericMaxKeys) * (sizeof(float) + sizeof(int));
  const unsigned blocks = static_cast<unsigned>(a.B) * a.T * a.H;
  if (a.dtype == 1)
    hipLaunchKernelGGL((attend_generic_kernel<bf16_t>), dim3(blocks), dim3(256), shmem, st, a);
  else
    hipLaunchKernelGGL((attend_generic_kernel<float>), dim3(blocks), dim3(256), shmem, st, a);
  return hipGetLastError();
}

}  // namespace dsv4
