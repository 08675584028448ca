// Compressor pooling (CSA overlapping windows / HCA disjoint windows) and the sliding-window
// RoPE copy, for gfx950.
//
// Source: DeepSeek-V4 model page (Transformers docs), "Hybrid attention (§2.3)" (CSA / HCA
// pools, sliding-window K=V branch, partial RoPE) and "Attention mask layout" (an entry covers
// the positions of its window and closes at the window's last token).
//
// Both kernels are HBM-bound streaming kernels: every thread owns VEC consecutive channels
// (16-byte loads for bf16 with VEC = 8) so that a wavefront reads whole contiguous rows.
#include "common.h"
#include "launch.h"

namespace dsv4 {

// ---------------------------------------------------------------------------
// compress: entry w, channel c = softmax_j(gate[j,c] + bias[slot,c]) weighted sum of x[j,c]
// over the window of w (reading R1/R2), then RoPE at (w+1)m - 1 (R5).
//
// Block layout: threads = E entries x P slot-groups x G channel-groups (G = C / VEC).
// Each thread runs an online softmax over its slot range; the P partial states of one
// (entry, channel group) are merged through LDS.  The online update uses one exp2 per
// element: of the old maximum and the new logit, exactly one is the new maximum.
// ---------------------------------------------------------------------------
template <typename T, int VEC>
__global__ void __launch_bounds__(256) compress_kernel(
    const T* __restrict__ x, const T* __restrict__ gate, const float* __restrict__ bias,
    T* __restrict__ pool, int S, int C, int m, int overlap, int e0, int e1, int N_cap, int r,
    double theta, long long pos_off, int G, int P, int E) {
  extern __shared__ float red[];  // [E*P*G][3*VEC] partial states when P > 1
  __shared__ double inv_freq[kMaxRope / 2];
  rope_table(inv_freq, r, theta);
  const int tid = threadIdx.x;
  const int g = tid % G;
  const int p = (tid / G) % P;
  const int e = tid / (G * P);
  const int b = blockIdx.y;
  const int w = e0 + blockIdx.x * E + e;
  const bool active = (e < E) && (w < e1);
  const int span = overlap ? 2 * m : m;
  const int lo = overlap ? (w - 1) * m : w * m;
  const int chunk = (span + P - 1) / P;
  const int s0 = p * chunk;
  const int s1 = min(span, s0 + chunk);
  const int c0 = g * VEC;

  float mx[VEC], sm[VEC], acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) { mx[i] = -INFINITY; sm[i] = 0.f; acc[i] = 0.f; }

  if (active) {
    const size_t row0 = static_cast<size_t>(b) * S;
    for (int s = s0; s < s1; ++s) {
      const int j = lo + s;
      if (j < 0 || j >= S) continue;
      float xv[VEC], gv[VEC];
      Chunk<T>::template load<VEC>(x + (row0 + j) * C + c0, xv);
      Chunk<T>::template load<VEC>(gate + (row0 + j) * C + c0, gv);
      if (bias != nullptr) {
        float bv[VEC];
        Chunk<float>::template load<VEC>(bias + static_cast<size_t>(s) * C + c0, bv);
#pragma unroll
        for (int i = 0; i < VEC; ++i) gv[i] += bv[i];
      }
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        const float a = gv[i] * kLog2e;
        const float d = exp2f(-fabsf(a - mx[i]));  // 0 on the first slot (mx = -inf)
        if (a > mx[i]) {
          sm[i] = sm[i] * d + 1.f;
          acc[i] = acc[i] * d + xv[i];
          mx[i] = a;
        } else {
          sm[i] += d;
          acc[i] += d * xv[i];
        }
      }
    }
  }

  __syncthreads();  // inv_freq ready
  if (P > 1) {
    float* mine = red + static_cast<size_t>(tid) * 3 * VEC;
#pragma unroll
    for (int i = 0; i < VEC; ++i) { mine[i] = mx[i]; mine[VEC + i] = sm[i]; mine[2 * VEC + i] = acc[i]; }
    __syncthreads();
    if (p == 0) {
      for (int q = 1; q < P; ++q) {
        const float* o = red + static_cast<size_t>(tid + q * G) * 3 * VEC;
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const float om = o[i];
          if (om == -INFINITY) continue;
          const float nm = fmaxf(mx[i], om);
          const float fa = exp2f(mx[i] - nm), fb = exp2f(om - nm);
          sm[i] = sm[i] * fa + o[VEC + i] * fb;
          acc[i] = acc[i] * fa + o[2 * VEC + i] * fb;
          mx[i] = nm;
        }
      }
    }
  }
  if (!active || p != 0) return;

  float out[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) out[i] = acc[i] / sm[i];
  const double pos = static_cast<double>((static_cast<long long>(w) + 1) * m - 1 + pos_off);
  rope_chunk<VEC>(out, c0, C, r, pos, inv_freq);
  Chunk<T>::template store<VEC>(pool + (static_cast<size_t>(b) * N_cap + w) * C + c0, out);
}

template <typename T, int VEC>
static hipError_t compress_t(const void* x, const void* gate, const float* bias, void* pool, int B,
                             int S, int C, int m, int overlap, int e0, int e1, int N_cap, int r,
                             double theta, long long off, hipStream_t st) {
  const int G = C / VEC;
  const int span = overlap ? 2 * m : m;
  int P = 1;
  if (span >= 32) P = max(1, min(256 / G, span / 16));
  int E = max(1, 256 / (G * P));
  const int threads = G * P * E;
  const int n = e1 - e0;
  if (n <= 0) return hipSuccess;
  dim3 grid(div_up(n, E), B);
  size_t shmem = P > 1 ? static_cast<size_t>(threads) * 3 * VEC * sizeof(float) : 0;
  hipLaunchKernelGGL((compress_kernel<T, VEC>), grid, dim3(threads), shmem, st,
                     static_cast<const T*>(x), static_cast<const T*>(gate), bias,
                     static_cast<T*>(pool), S, C, m, overlap, e0, e1, N_cap, r, theta, off, G, P, E);
  return hipGetLastError();
}

hipError_t launch_compress(const void* x, const void* gate, const float* bias, void* pool, int B,
                           int S, int C, int m, int overlap, int e0, int e1, int N_cap, int r,
                           double theta, long long off, int dtype, hipStream_t st) {
  const bool v8 = (C % 8 == 0) && (C / 8 <= 256);
  if (dtype == 1) {
    return v8 ? compress_t<bf16_t, 8>(x, gate, bias, pool, B, S, C, m, overlap, e0, e1, N_cap, r, theta, off, st)
              : compress_t<bf16_t, 2>(x, gate, bias, pool, B, S, C, m, overlap, e0, e1, N_cap, r, theta, off, st);
  }
  return v8 ? compress_t<float, 8>(x, gate, bias, pool, B, S, C, m, overlap, e0, e1, N_cap, r, theta, off, st)
            : compress_t<float, 2>(x, gate, bias, pool, B, S, C, m, overlap, e0, e1, N_cap, r, theta, off, st);
}

// ---------------------------------------------------------------------------
// swa_concat: rotate raw K=V rows at their positions into the window buffer.
// One thread per VEC-channel chunk of one row.
// ---------------------------------------------------------------------------
template <typename T, int VEC>
__global__ void __launch_bounds__(256) swa_kernel(const T* __restrict__ kv_raw, T* kv_win,
                                                  const int* __restrict__ kv_pos0,
                                                  const int* __restrict__ new_pos0, int S_new,
                                                  int S_cap, int D, int r, double theta,
                                                  long long pos_off, long long total) {
  __shared__ double inv_freq[kMaxRope / 2];
  rope_table(inv_freq, r, theta);
  __syncthreads();
  const long long gid = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int G = D / VEC;
  const int g = static_cast<int>(gid % G);
  const long long row = gid / G;  // b * S_new + i
  const int i = static_cast<int>(row % S_new);
  const int b = static_cast<int>(row / S_new);
  const long long seq = static_cast<long long>(new_pos0[b]) + i;
  const long long dst = seq - kv_pos0[b];
  if (dst < 0 || dst >= S_cap) return;
  float v[VEC];
  Chunk<T>::template load<VEC>(kv_raw + row * D + g * VEC, v);
  rope_chunk<VEC>(v, g * VEC, D, r, static_cast<double>(seq + pos_off), inv_freq);
  Chunk<T>::template store<VEC>(kv_win + (static_cast<long long>(b) * S_cap + dst) * D + g * VEC, v);
}

template <typename T, int VEC>
static hipError_t swa_t(const void* kv_raw, void* kv_win, const int* kv_pos0, const int* new_pos0,
                        int B, int S_new, int S_cap, int D, int r, double theta, long long off,
                        hipStream_t st) {
  const long long total = static_cast<long long>(B) * S_new * (D / VEC);
  if (total == 0) return hipSuccess;
  const int threads = 256;
  hipLaunchKernelGGL((swa_kernel<T, VEC>), dim3(static_cast<unsigned>((total + threads - 1) / threads)),
                     dim3(threads), 0, st, static_cast<const T*>(kv_raw), static_cast<T*>(kv_win),
                     kv_pos0, new_pos0, S_new, S_cap, D, r, theta, off, total);
  return hipGetLastError();
}

hipError_t launch_swa(const void* kv_raw, void* kv_win, const int* kv_pos0, const int* new_pos0,
                      int B, int S_new, int S_cap, int D, int r, double theta, long long off,
                      int dtype, hipStream_t st) {
  const bool v8 = (D % 8 == 0);
  if (dtype == 1)
    return v8 ? swa_t<bf16_t, 8>(kv_raw, kv_win, kv_pos0, new_pos0, B, S_new, S_cap, D, r, theta, off, st)
              : swa_t<bf16_t, 2>(kv_raw, kv_win, kv_pos0, new_pos0, B, S_new, S_cap, D, r, theta, off, st);
  return v8 ? swa_t<float, 8>(kv_raw, kv_win, kv_pos0, new_pos0, B, S_new, S_cap, D, r, theta, off, st)
            : swa_t<float, 2>(kv_raw, kv_win, kv_pos0, new_pos0, B, S_new, S_cap, D, r, theta, off, st);
}

}  // namespace dsv4
