// Dense products C = A . B^T for the projections around the attention core, on MFMA for
// gfx950 (bf16 storage, fp32 accumulation), with a plain fallback for other shapes.
//
// Source: DeepSeek-V4 model page (Transformers docs), "Hybrid attention (§2.3)", grouped output
// projection item (o_groups head groups -> o_lora_rank per group -> hidden_size: a grouped
// linear o_a_proj followed by o_b_proj) and "DeepseekV4Config" (o_groups, o_lora_rank,
// hidden_size).  Both factors are dense contractions: the grouped one is a batch of o_groups
// independent products (one per head group), the second a single product.
//
// The layer's input projections are the same kind of product: several linear maps of one
// input, whose weights stacked row-wise make one B, so one launch fills the chip where the
// narrow ones alone (64 or 128 columns) would not.  The columns of C then split into
// segments, each stored in its own buffer and type (the indexer head weights in fp32).
//
// Operands: A [M, K] rows of stride lda, B [N, K] rows of stride ldb (a linear layer's
// [out, in] weight), C's column segments as described by GemmOut; batch g offsets A, B and
// each segment by sA, sB and the segment's stride.  Both factors are K-contiguous, so their
// tiles move and are read the same way.
//
// bf16 path (K % 64 == 0, every output segment a multiple of 32 columns wide):
//   * one 256 x 256 tile of C per workgroup, four waves of 128 x 128 (one per SIMD), 64-deep
//     K steps on v_mfma_f32_32x32x16_bf16; the accumulators (256 per lane) sit in the
//     accumulator registers;
//   * tiles move from global memory straight into LDS with buffer_load ... lds, two stages
//     of 64 KB; the next step's 16 loads per wave are spread over the first 32 of this
//     step's 64 matrix instructions (one every two), which measured faster than issuing them
//     in one burst or over the whole step (L2 -> LDS fill, ~45 B/clk per CU, is the limit:
//     a step needs 64 KB per 2048 matrix cycles).  Each 128-byte tile row keeps its 16-byte
//     chunks XOR-swizzled (chunk c of row r at c ^ ((r >> 1) & 7), applied on the load
//     side), so the 32-row fragment reads are conflict-free;
//   * the wave computes C^T blocks (A's fragment as the B operand), so that each lane holds
//     4 consecutive output columns per group and a 32-lane swap makes 16-byte stores;
//   * rows at or beyond M (and B rows at or beyond N in a ragged last tile column) read
//     zeros; their stores are skipped.
#include "common.h"
#include "launch.h"

namespace dsv4 {

typedef __attribute__((ext_vector_type(8))) __bf16 gbf16x8_t;
typedef __attribute__((ext_vector_type(16))) float gf32x16_t;
typedef __attribute__((ext_vector_type(4))) float gf32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned gu32x4_t;

namespace {

constexpr int GM = 256, GN = 256, GK = 64;  // workgroup tile
constexpr int GROW = GK * 2;                // LDS bytes per tile row (128)
constexpr int GTILE = GM * GROW;            // bytes per operand tile (32 KB)
constexpr int kGemmLds = 2 * 2 * GTILE;     // [stage][A | B]

typedef __attribute__((address_space(3))) void glds_void;
typedef __amdgpu_buffer_rsrc_t grsrc_t;

__device__ __forceinline__ grsrc_t gmake_rs(const void* base, unsigned long long bytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  const unsigned lo = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(a));
  const unsigned hi = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(a >> 32));
  const unsigned n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : static_cast<unsigned>(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((static_cast<unsigned long long>(hi) << 32) | lo),
                                           static_cast<short>(0), static_cast<int>(__builtin_amdgcn_readfirstlane(n)),
                                           0x00020000);
}

__device__ __forceinline__ int gswz(int row) { return (row >> 1) & 7; }

}  // namespace

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_bt_mfma(const bf16_t* __restrict__ A, const bf16_t* __restrict__ B, const GemmOut out, int M, int N, int K,
             long long lda, long long ldb, long long sA, long long sB, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) unsigned char glds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Tile order: workgroups are dealt to the 8 XCDs round-robin, so each XCD takes a
  // contiguous range of tile ranks (when the count divides), walked kGroup tile rows at a
  // time: the workgroups that run together on one XCD then share few A and B tiles in its
  // L2 (measured ~8 % faster on the output projection than row-major ranks).
  int tm, tn;
  {
    constexpr int kGroup = 4;
    const int n_t = static_cast<int>(gridDim.x);
    const int bid = static_cast<int>(blockIdx.x);
    const int rank = (n_t % 8 == 0) ? (bid % 8) * (n_t / 8) + bid / 8 : bid;
    const int tiles_m = n_t / tiles_n;
    const int grp = kGroup * tiles_n;
    const int first_m = (rank / grp) * kGroup;
    const int gsz = tiles_m - first_m < kGroup ? tiles_m - first_m : kGroup;
    tm = first_m + (rank % grp) % gsz;
    tn = (rank % grp) / gsz;
  }
  const int g = blockIdx.y;
  const int m0 = tm * GM, n0 = tn * GN;
  // operand descriptors of this batch entry; A covers rows 0..M-1 only (later rows read 0)
  const bf16_t* Ab = A + g * sA;
  const bf16_t* Bb = B + g * sB;
  const grsrc_t a_rs = gmake_rs(Ab + static_cast<long long>(m0) * lda,
                                static_cast<unsigned long long>(M - m0) * lda * 2);
  // B covers rows n0 .. N-1 of this tile column only (a ragged last column reads zeros)
  const grsrc_t b_rs = gmake_rs(Bb + static_cast<long long>(n0) * ldb,
                                static_cast<unsigned long long>(N - n0 < GN ? N - n0 : GN) * ldb * 2);
  // Load lanes: per K step each operand tile is 32 loads of 1 KB (8 rows x 128 bytes); wave w
  // issues loads 8w .. 8w + 7 of each.  Lane l fills LDS chunk l % 8 of row 8 i + l / 8 with
  // the global chunk (l % 8) ^ swz(row).
  unsigned a_off[8], b_off[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 8 * (8 * wave + i) + (lane >> 3);
    const int c = (lane & 7) ^ gswz(r);
    a_off[i] = static_cast<unsigned>(r * lda * 2 + c * 16);
    b_off[i] = static_cast<unsigned>(r * ldb * 2 + c * 16);
  }
  auto issue = [&](int j, int ks, int stage) {  // load j (0..15: A then B) of K step ks
    const int i = j & 7;
    unsigned char* dst = glds + stage * 2 * GTILE + (j >> 3) * GTILE + (8 * (8 * wave + i)) * GROW;
    const unsigned soff = static_cast<unsigned>(ks * GK * 2);
    if (j < 8)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rs, (glds_void*)dst, 16, a_off[i], soff, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rs, (glds_void*)dst, 16, b_off[i], soff, 0, 0);
  };
  // Fragment reads: row (32 block + lane % 32) of a 128-row half, chunk 2 kk + lane / 32.
  const int wm = wave & 1, wn = wave >> 1;
  const int l32 = lane & 31, half = lane >> 5;
  int fr_off[4];  // byte offset of block i's row in the A (wm) / B (wn) half, swizzle folded in
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 32 * i + l32;  // swz depends on r's bits 1..3 only: the same for +128
    fr_off[i] = r * GROW + ((half ^ gswz(r)) << 4);
  }
  gf32x16_t acc[4][4];  // [n block][m block] of C^T
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  const int n_ks = K / GK;
#pragma unroll
  for (int j = 0; j < 16; ++j) issue(j, 0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  for (int ks = 0; ks < n_ks; ++ks) {
    const int st = ks & 1;
    const bool more = ks + 1 < n_ks;
    const unsigned char* sa = glds + st * 2 * GTILE + wm * 128 * GROW;
    const unsigned char* sb = glds + st * 2 * GTILE + GTILE + wn * 128 * GROW;
    // fragments of 16-deep step kk, double-buffered; chunk 2 kk + half of row r sits at
    // (2 kk + half) ^ swz(r) = (half ^ swz(r)) ^ 2 kk
    gbf16x8_t af[2][4], bfr[2][4];
    auto frags = [&](int kk, int b) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[b][i] = *reinterpret_cast<const gbf16x8_t*>(sa + (fr_off[i] ^ (32 * kk)));
        bfr[b][i] = *reinterpret_cast<const gbf16x8_t*>(sb + (fr_off[i] ^ (32 * kk)));
      }
    };
    
    frags(0, 0);
#pragma unroll
    for (int kk = 0; kk < GK / 16; ++kk) {
      const int b = kk & 1;
      if (kk + 1 < GK / 16) frags(kk + 1, b ^ 1);
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        acc[t >> 2][t & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[b][t >> 2], af[b][t & 3], acc[t >> 2][t & 3], 0, 0, 0);
        if (kk < 2 && (t & 1) && more) issue(kk * 8 + (t >> 1), ks + 1, st ^ 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of step ks + 1 landed
    __syncthreads();                     // every wave's loads landed, stage st is free again
  }

  // epilogue: C^T block (ni, mi) holds, for output row m = m0 + 128 wm + 32 mi + l32, columns
  // nb + 8 q + 4 half + 0..3 (q = 0..3), nb = n0 + 128 wn + 32 ni.  Segment bounds are
  // multiples of 32, so a block lies in one output segment, looked up once per block.  bf16:
  // a 32-lane swap gives each lane 8 consecutive columns (one 16-byte store per 16 columns);
  // fp32: each lane stores its own 4-column runs.
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    const int nb = n0 + 128 * wn + 32 * ni;
    if (nb >= N) break;
    int s = 0;
#pragma unroll
    for (int i = 1; i < kGemmMaxSeg; ++i) s += (i < out.n_seg && nb >= out.begin[i]) ? 1 : 0;
    s = __builtin_amdgcn_readfirstlane(s);
    const int col = nb - out.begin[s];
    const bool f32 = out.f32[s] != 0;
    const long long ld = out.ld[s];
    const int esz = f32 ? 4 : 2;
    const unsigned char* cbase = static_cast<const unsigned char*>(out.ptr[s]) +
                                 (g * out.stride[s] + static_cast<long long>(m0) * ld) * esz;
    const grsrc_t c_rs = gmake_rs(cbase, static_cast<unsigned long long>(M - m0) * ld * esz);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int ml = 128 * wm + 32 * mi + l32;  // row within the tile
      const bool live = m0 + ml < M;
      const unsigned row_off = static_cast<unsigned>(static_cast<long long>(ml) * ld * esz);
      if (f32) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const gf32x4_t v4 = {acc[ni][mi][4 * q], acc[ni][mi][4 * q + 1], acc[ni][mi][4 * q + 2],
                               acc[ni][mi][4 * q + 3]};
          const gu32x4_t val = __builtin_bit_cast(gu32x4_t, v4);
          if (live)
            __builtin_amdgcn_raw_buffer_store_b128(val, c_rs, row_off + static_cast<unsigned>(col + 8 * q + 4 * half) * 4,
                                                   0, 0);
        }
        continue;
      }
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        unsigned w[2][2];
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
          const int q = 2 * gp + g2;
          w[g2][0] = pack_bf16x2(acc[ni][mi][4 * q], acc[ni][mi][4 * q + 1]);
          w[g2][1] = pack_bf16x2(acc[ni][mi][4 * q + 2], acc[ni][mi][4 * q + 3]);
        }
        const auto s0 = __builtin_amdgcn_permlane32_swap(w[0][0], w[1][0], false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(w[0][1], w[1][1], false, false);
        gu32x4_t val;
        val[0] = s0[0];
        val[1] = s1[0];
        val[2] = s0[1];
        val[3] = s1[1];
        // lanes < 32 write columns 16 gp + 0..7 of the block, lanes >= 32 columns 16 gp + 8..15
        if (live)
          __builtin_amdgcn_raw_buffer_store_b128(val, c_rs, row_off + static_cast<unsigned>(col + 16 * gp + 8 * half) * 2,
                                                 0, 0);
      }
    }
  }
}

// Any shape, bf16 or fp32 storage, fp32 accumulation: one thread per output element.
template <typename T>
__global__ void __launch_bounds__(256) gemm_bt_generic(const T* __restrict__ A, const T* __restrict__ B,
                                                       const GemmOut out, int M, int N, int K, long long lda,
                                                       long long ldb, long long sA, long long sB) {
  const long long idx = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  const int g = blockIdx.y;
  if (idx >= static_cast<long long>(M) * N) return;
  const int m = static_cast<int>(idx / N), n = static_cast<int>(idx % N);
  const T* a = A + g * sA + m * lda;
  const T* b = B + g * sB + n * ldb;
  float acc = 0.f;
  for (int k = 0; k < K; ++k) {
    float x, y;
    if constexpr (sizeof(T) == 2) {
      x = bf16_to_f32(a[k]);
      y = bf16_to_f32(b[k]);
    } else {
      x = a[k];
      y = b[k];
    }
    acc = fmaf(x, y, acc);
  }
  int s = 0;
  for (int i = 1; i < out.n_seg; ++i) s += n >= out.begin[i] ? 1 : 0;
  const long long off = g * out.stride[s] + m * out.ld[s] + (n - out.begin[s]);
  if (out.f32[s]) static_cast<float*>(out.ptr[s])[off] = acc;
  else static_cast<bf16_t*>(out.ptr[s])[off] = f32_to_bf16(acc);
}

bool gemm_fast(const GemmOut& out, int K, long long lda, long long ldb, int dtype) {
  // 16-byte operand rows and in-tile byte offsets that fit 32 bits
  if (dtype != 1 || K % GK != 0 || lda % 8 != 0 || ldb % 8 != 0 || lda > (1 << 22) || ldb > (1 << 22)) return false;
  for (int s = 0; s < out.n_seg; ++s) {
    const int per16 = out.f32[s] ? 4 : 8;  // elements per 16 bytes
    if ((out.begin[s + 1] - out.begin[s]) % 32 != 0 || out.ld[s] % per16 != 0 || out.stride[s] % per16 != 0 ||
        out.ld[s] > (1 << 21))
      return false;
  }
  return true;
}

hipError_t launch_gemm_bt_seg(const void* A, const void* B, const GemmOut& out, int M, int K, long long lda,
                              long long ldb, int batch, long long sA, long long sB, int dtype, hipStream_t st) {
  const int N = out.begin[out.n_seg];
  if (M == 0 || N == 0 || batch == 0) return hipSuccess;
  if (gemm_fast(out, K, lda, ldb, dtype)) {
    static bool attr_set = false;
    if (!attr_set) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_bt_mfma),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
      if (e != hipSuccess) return e;
      attr_set = true;
    }
    const int tiles_m = (M + GM - 1) / GM, tiles_n = (N + GN - 1) / GN;
    hipLaunchKernelGGL(gemm_bt_mfma, dim3(tiles_m * tiles_n, batch), dim3(256), kGemmLds, st,
                       static_cast<const bf16_t*>(A), static_cast<const bf16_t*>(B), out, M, N, K, lda, ldb, sA, sB,
                       tiles_n);
    return hipGetLastError();
  }
  const long long total = static_cast<long long>(M) * N;
  const dim3 grid(static_cast<unsigned>((total + 255) / 256), batch);
  if (dtype == 1)
    hipLaunchKernelGGL(gemm_bt_generic<bf16_t>, grid, dim3(256), 0, st, static_cast<const bf16_t*>(A),
                       static_cast<const bf16_t*>(B), out, M, N, K, lda, ldb, sA, sB);
  else
    hipLaunchKernelGGL(gemm_bt_generic<float>, grid, dim3(256), 0, st, static_cast<const float*>(A),
                       static_cast<const float*>(B), out, M, N, K, lda, ldb, sA, sB);
  return hipGetLastError();
}

hipError_t launch_gemm_bt(const void* A, const void* B, void* C, int M, int N, int K, long long lda,
                          long long ldb, long long ldc, int batch, long long sA, long long sB, long long sC,
                          int dtype, hipStream_t st) {
  GemmOut out{};
  out.n_seg = 1;
  out.begin[0] = 0;
  out.begin[1] = N;
  out.f32[0] = dtype == 0;
  out.ld[0] = ldc;
  out.stride[0] = sC;
  out.ptr[0] = C;
  return launch_gemm_bt_seg(A, B, out, M, K, lda, ldb, batch, sA, sB, dtype, st);
}

}  // namespace dsv4
