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
    const T* __restrict__ x, const T* __restrict__ gate, const T* __restrict__ x_prev,
    const T* __restrict__ gate_prev, const float* __restrict__ bias, T* __restrict__ pool, int S,
    int C, int m, int overlap, int e0, int e1, int N_cap, int r, const RopeFreq rf, long long pos_off,
    int G, int P, int E) {
  extern __shared__ float red[];  // [E*P*G][3*VEC] partial states when P > 1
  __shared__ double inv_freq[kMaxRope / 2];
  for (int i = threadIdx.x; i < r / 2; i += blockDim.x) inv_freq[i] = rf.inv[i];
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
    // Slots in groups of U: the row loads of a group (values, gates and the slot biases) are
    // all issued before any is used, so a thread keeps them in flight together instead of
    // paying one slot's latency at a time (a bias load issued at its use would make the wait
    // for it cover every load issued before it).
    constexpr int U = 8;
    for (int sg = s0; sg < s1; sg += U) {
      float xv[U][VEC], gv[U][VEC], bv[U][VEC];
      bool ok[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int s = sg + u;
        const int j = lo + s;
        ok[u] = s < s1 && j >= 0 && j < S;
        const size_t jr = row0 + (ok[u] ? j : 0);  // a valid row; unused when !ok
        // the earlier half of a window reads the second projection when one is given
        const bool early = x_prev != nullptr && s < m;
        Chunk<T>::template load<VEC>((early ? x_prev : x) + jr * C + c0, xv[u]);
        Chunk<T>::template load<VEC>((early ? gate_prev : gate) + jr * C + c0, gv[u]);
        if (bias != nullptr)
          Chunk<float>::template load<VEC>(bias + static_cast<size_t>(ok[u] ? s : 0) * C + c0, bv[u]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (!ok[u]) continue;
        if (bias != nullptr) {
#pragma unroll
          for (int i = 0; i < VEC; ++i) gv[u][i] += bv[u][i];
        }
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const float a = gv[u][i] * kLog2e;
          const float d = exp2f(-fabsf(a - mx[i]));  // 0 on the first slot (mx = -inf)
          if (a > mx[i]) {
            sm[i] = sm[i] * d + 1.f;
            acc[i] = acc[i] * d + xv[u][i];
            mx[i] = a;
          } else {
            sm[i] += d;
            acc[i] += d * xv[u][i];
          }
        }
      }
    }
  }

  __syncthreads();  // inv_freq staged
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
  rope_chunk<VEC, sizeof(T) == 2>(out, c0, C, r, pos, inv_freq);
  Chunk<T>::template store<VEC>(pool + (static_cast<size_t>(b) * N_cap + w) * C + c0, out);
}

template <typename T, int VEC>
static hipError_t compress_t(const void* x, const void* gate, const void* x_prev, const void* gate_prev,
                             const float* bias, void* pool, int B, int S, int C, int m, int overlap, int e0,
                             int e1, int N_cap, int r, double theta, long long off, hipStream_t st) {
  const int G = C / VEC;
  const int span = overlap ? 2 * m : m;
  // long windows: split the slots over P thread groups (16+ slots each)
  int P = 1;
  if (span >= 32) P = max(1, min(256 / G, span / 16));
  const int E = max(1, 256 / (G * P));
  const int threads = G * P * E;
  const int n = e1 - e0;
  if (n <= 0) return hipSuccess;
  dim3 grid(div_up(n, E), B);
  size_t shmem = P > 1 ? static_cast<size_t>(threads) * 3 * VEC * sizeof(float) : 0;
  hipLaunchKernelGGL((compress_kernel<T, VEC>), grid, dim3(threads), shmem, st,
                     static_cast<const T*>(x), static_cast<const T*>(gate), static_cast<const T*>(x_prev),
                     static_cast<const T*>(gate_prev), bias, static_cast<T*>(pool), S, C, m, overlap, e0, e1,
                     N_cap, r,
                     make_rope_freq(r, theta), off, G, P, E);
  return hipGetLastError();
}

hipError_t launch_compress(const void* x, const void* gate, const void* x_prev, const void* gate_prev,
                           const float* bias, void* pool, int B, int S, int C, int m, int overlap, int e0,
                           int e1, int N_cap, int r, double theta, long long off, int dtype, hipStream_t st) {
  const bool v8 = (C % 8 == 0) && (C / 8 <= 256);
  if (!overlap) x_prev = gate_prev = nullptr;  // no earlier half
  if (dtype == 1) {
    return v8 ? compress_t<bf16_t, 8>(x, gate, x_prev, gate_prev, bias, pool, B, S, C, m, overlap, e0, e1, N_cap, r,
                                      theta, off, st)
              : compress_t<bf16_t, 2>(x, gate, x_prev, gate_prev, bias, pool, B, S, C, m, overlap, e0, e1, N_cap, r,
                                      theta, off, st);
  }
  return v8 ? compress_t<float, 8>(x, gate, x_prev, gate_prev, bias, pool, B, S, C, m, overlap, e0, e1, N_cap, r,
                                   theta, off, st)
            : compress_t<float, 2>(x, gate, x_prev, gate_prev, bias, pool, B, S, C, m, overlap, e0, e1, N_cap, r,
                                   theta, off, st);
}

// ---------------------------------------------------------------------------
// Compressor cache update (decode): one workgroup per sequence.  lengths[b] = L counts the
// sequence's tokens including the new one.  The new raw token (x_new[b], gate_new[b]) goes
// into ring slot (L-1) mod span of the sequence's token ring (span = 2m with overlap, m
// without); when it closes an entry (L mod m == 0, emit != 0), entry w = L/m - 1 is pooled
// from the ring exactly as compress_kernel pools it with P = 1 (same slot order, same
// online softmax) and rotated at (w+1)m - 1.  Each thread owns one channel chunk of both the
// store and the pooling, so it reads back its own write.
// ---------------------------------------------------------------------------
template <typename T, int VEC>
__global__ void __launch_bounds__(256) cache_update_kernel(
    const T* __restrict__ x_new, const T* __restrict__ g_new, T* x_ring, T* g_ring,
    const T* __restrict__ xp_new, const T* __restrict__ gp_new, T* xp_ring, T* gp_ring,
    const float* __restrict__ bias, T* __restrict__ pool, const int* __restrict__ lengths, int C,
    int m, int overlap, int N_cap, int r, const RopeFreq rf, long long pos_off, int emit) {
  __shared__ double inv_freq[kMaxRope / 2];
  for (int i = threadIdx.x; i < r / 2; i += blockDim.x) inv_freq[i] = rf.inv[i];
  __syncthreads();
  const int b = blockIdx.x;
  const int L = lengths[b];
  if (L < 1) return;  // block-uniform; no barrier follows
  const int span = overlap ? 2 * m : m;
  const int G = C / VEC;
  const size_t ring0 = static_cast<size_t>(b) * span;
  const int slot = (L - 1) % span;
  const bool closes = emit && (L % m) == 0 && (L / m - 1) < N_cap;
  const int w = L / m - 1;
  const int lo = overlap ? (w - 1) * m : w * m;
  for (int g = threadIdx.x; g < G; g += blockDim.x) {
    const int c0 = g * VEC;
    float v[VEC];
    Chunk<T>::template load<VEC>(x_new + static_cast<size_t>(b) * C + c0, v);
    Chunk<T>::template store<VEC>(x_ring + (ring0 + slot) * C + c0, v);
    Chunk<T>::template load<VEC>(g_new + static_cast<size_t>(b) * C + c0, v);
    Chunk<T>::template store<VEC>(g_ring + (ring0 + slot) * C + c0, v);
    if (xp_ring != nullptr) {  // the second projection, for the windows this token starts
      Chunk<T>::template load<VEC>(xp_new + static_cast<size_t>(b) * C + c0, v);
      Chunk<T>::template store<VEC>(xp_ring + (ring0 + slot) * C + c0, v);
      Chunk<T>::template load<VEC>(gp_new + static_cast<size_t>(b) * C + c0, v);
      Chunk<T>::template store<VEC>(gp_ring + (ring0 + slot) * C + c0, v);
    }
    if (!closes) continue;
    float mx[VEC], sm[VEC], acc[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) { mx[i] = -INFINITY; sm[i] = 0.f; acc[i] = 0.f; }
    for (int s = 0; s < span; ++s) {
      const int p = lo + s;  // token position; absent before 0
      if (p < 0) continue;
      const size_t row = ring0 + p % span;
      float xv[VEC], gv[VEC];
      const bool early = xp_ring != nullptr && s < m;  // the earlier half's second projection
      Chunk<T>::template load<VEC>((early ? xp_ring : x_ring) + row * C + c0, xv);
      Chunk<T>::template load<VEC>((early ? gp_ring : g_ring) + row * C + c0, gv);
      if (bias != nullptr) {
        float bv[VEC];
        Chunk<float>::template load<VEC>(bias + static_cast<size_t>(s) * C + c0, bv);
#pragma unroll
        for (int i = 0; i < VEC; ++i) gv[i] += bv[i];
      }
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        const float a = gv[i] * kLog2e;
        const float d = exp2f(-fabsf(a - mx[i]));
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
    float out[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) out[i] = acc[i] / sm[i];
    const double pos = static_cast<double>((static_cast<long long>(w) + 1) * m - 1 + pos_off);
    rope_chunk<VEC, sizeof(T) == 2>(out, c0, C, r, pos, inv_freq);
    Chunk<T>::template store<VEC>(pool + (static_cast<size_t>(b) * N_cap + w) * C + c0, out);
  }
}

template <typename T, int VEC>
static hipError_t cache_update_t(const CacheUpdate& u, int B, int C, int m, int overlap, int N_cap, int r,
                                 double theta, long long off, int emit, hipStream_t st) {
  const int G = C / VEC;
  const int threads = G >= 256 ? 256 : ((G + 63) / 64) * 64;
  hipLaunchKernelGGL((cache_update_kernel<T, VEC>), dim3(B), dim3(threads), 0, st,
                     static_cast<const T*>(u.x_new), static_cast<const T*>(u.g_new), static_cast<T*>(u.x_ring),
                     static_cast<T*>(u.g_ring), static_cast<const T*>(u.xp_new), static_cast<const T*>(u.gp_new),
                     static_cast<T*>(u.xp_ring), static_cast<T*>(u.gp_ring), u.bias, static_cast<T*>(u.pool),
                     u.lengths, C, m, overlap, N_cap, r, make_rope_freq(r, theta), off, emit);
  return hipGetLastError();
}

hipError_t launch_cache_update(const CacheUpdate& u, int B, int C, int m, int overlap, int N_cap, int r,
                               double theta, long long off, int emit, int dtype, hipStream_t st) {
  if (B == 0) return hipSuccess;
  CacheUpdate v = u;
  if (!overlap || v.xp_ring == nullptr) v.xp_new = v.gp_new = v.xp_ring = v.gp_ring = nullptr;
  const bool v8 = (C % 8 == 0) && (C / 8 <= 256);
  if (dtype == 1)
    return v8 ? cache_update_t<bf16_t, 8>(v, B, C, m, overlap, N_cap, r, theta, off, emit, st)
              : cache_update_t<bf16_t, 2>(v, B, C, m, overlap, N_cap, r, theta, off, emit, st);
  return v8 ? cache_update_t<float, 8>(v, B, C, m, overlap, N_cap, r, theta, off, emit, st)
            : cache_update_t<float, 2>(v, B, C, m, overlap, N_cap, r, theta, off, emit, st);
}

// ---------------------------------------------------------------------------
// swa_concat: rotate raw K=V rows at their positions into the window buffer.
//
// The chunks of a row that hold no rotary channel (the first Gn of its G VEC-channel chunks)
// are a plain copy; the Gr = G - Gn trailing ones are rotated.  The grid is split in two
// regions so that no wavefront mixes the two kinds: blocks below nb_copy copy, the rest
// rotate (inv_freq staged in LDS).  Each thread handles SWA_U chunks a block-stride apart and
// issues all their loads before any store.  Index arithmetic is 32-bit (the host checks the
// chunk counts): 64-bit division is a long software sequence on this target.
// ---------------------------------------------------------------------------
constexpr int SWA_U = 4;

template <typename T, int VEC>
__global__ void __launch_bounds__(256) swa_kernel(const T* __restrict__ kv_raw, T* kv_win,
                                                  const int* __restrict__ kv_pos0,
                                                  const int* __restrict__ new_pos0, int S_new,
                                                  int S_cap, int D, int r, const RopeFreq rf,
                                                  long long pos_off, int Gn, unsigned n_copy,
                                                  unsigned n_rot, unsigned nb_copy) {
  __shared__ double inv_freq[kMaxRope / 2];
  const unsigned G = static_cast<unsigned>(D / VEC);
  const bool rot = blockIdx.x >= nb_copy;  // block-uniform
  const unsigned Gk = rot ? G - Gn : Gn;   // chunks of this kind per row
  const unsigned total = rot ? n_rot : n_copy;
  const unsigned blk = rot ? blockIdx.x - nb_copy : blockIdx.x;
  if (rot) {
    for (int i = threadIdx.x; i < r / 2; i += blockDim.x) inv_freq[i] = rf.inv[i];
    __syncthreads();
  }
  const unsigned base = blk * blockDim.x * SWA_U + threadIdx.x;
  float v[SWA_U][VEC];
#pragma unroll
  for (int u = 0; u < SWA_U; ++u) {
    const unsigned gid = base + u * blockDim.x;
    const unsigned ld = gid < total ? gid : total - 1;  // a valid chunk; unused past the end
    const unsigned row = ld / Gk;
    const unsigned g = (rot ? Gn : 0) + (ld - row * Gk);
    Chunk<T>::template load<VEC>(kv_raw + (static_cast<size_t>(row) * G + g) * VEC, v[u]);
  }
#pragma unroll
  for (int u = 0; u < SWA_U; ++u) {
    const unsigned gid = base + u * blockDim.x;
    if (gid >= total) break;
    const unsigned row = gid / Gk;  // b * S_new + i
    const int g = static_cast<int>((rot ? Gn : 0) + (gid - row * Gk));
    const int b = static_cast<int>(row / static_cast<unsigned>(S_new));
    const int i = static_cast<int>(row - static_cast<unsigned>(b) * S_new);
    const long long seq = static_cast<long long>(new_pos0[b]) + i;
    const long long dst = seq - kv_pos0[b];
    if (dst < 0 || dst >= S_cap) continue;
    if (rot)
      rope_chunk<VEC, sizeof(T) == 2>(v[u], g * VEC, D, r, static_cast<double>(seq + pos_off),
                                      inv_freq);
    Chunk<T>::template store<VEC>(kv_win + (static_cast<long long>(b) * S_cap + dst) * D + g * VEC,
                                  v[u]);
  }
}

template <typename T, int VEC>
static hipError_t swa_t(const void* kv_raw, void* kv_win, const int* kv_pos0, const int* new_pos0,
                        int B, int S_new, int S_cap, int D, int r, double theta, long long off,
                        hipStream_t st) {
  const long long rows = static_cast<long long>(B) * S_new;
  const int G = D / VEC;
  const int Gn = (D - r) / VEC;  // chunks with no rotary channel
  const long long n_copy = rows * Gn, n_rot = rows * (G - Gn);
  if (rows == 0) return hipSuccess;
  if (rows * G >= (1LL << 31)) return hipErrorInvalidValue;  // 32-bit chunk indices
  const int threads = 256;
  const long long per_block = static_cast<long long>(threads) * SWA_U;
  const long long nb_copy = (n_copy + per_block - 1) / per_block;
  const long long nb_rot = (n_rot + per_block - 1) / per_block;
  hipLaunchKernelGGL((swa_kernel<T, VEC>), dim3(static_cast<unsigned>(nb_copy + nb_rot)),
                     dim3(threads), 0, st, static_cast<const T*>(kv_raw), static_cast<T*>(kv_win),
                     kv_pos0, new_pos0, S_new, S_cap, D, r, make_rope_freq(r, theta), off, Gn,
                     static_cast<unsigned>(n_copy), static_cast<unsigned>(n_rot),
                     static_cast<unsigned>(nb_copy));
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
