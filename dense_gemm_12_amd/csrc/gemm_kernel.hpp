// The GEMM kernel template for gfx950: C = alpha * op(A) * op(B) + beta * C.
//
// Work decomposition ("SGEMM CUDA代码学习" steps 1-4 and "CUDA GEMM：从基础写法到
// 工程优化" sections 3, 10 and 11 describe the same hierarchy for NVIDIA parts;
// the sizes and instruction choices here are CDNA4's own):
//   * a workgroup of 4 waves (wave64) owns a BM x BN tile of C and walks K in
//     BK-deep slices;
//   * each slice of op(A) (BM x BK) and op(B)^T (BN x BK) is staged from HBM
//     into LDS, always as [row][k] with k contiguous, through 16-byte buffer
//     loads; a k-major operand (A stored K x M, or B stored K x N) is
//     transposed in registers on the way, so the MFMA feed never strides;
//   * LDS rows are 128 bytes with the 16-byte chunk index XORed with
//     (row mod 8): measured on gfx950, this keeps both the ds_write_b128 of
//     the staging (8 lanes per 128-byte row) and the ds_read_b128 fragment
//     reads (16 rows, one chunk per quarter-wave) free of bank conflicts,
//     where a 16-byte row pad still conflicts 2-way on the reads;
//   * two LDS buffers alternate: while the waves run MFMAs on slice k the
//     global loads for slice k+1 are in flight in registers, and one barrier
//     per slice separates the buffer swap ("SGEMM CUDA代码学习" step 4; the
//     worklog's closing notes on double buffering);
//   * each wave owns a (BM/WAVES_M) x (BN/WAVES_N) sub-tile as a grid of
//     16x16 MFMA blocks with fp32 accumulators in registers;
//   * the epilogue applies alpha and beta in fp32, rounds once to the output
//     type and masks every row/column tail.
// The MFMA is issued with the B-side chunk as its first operand, so each lane
// ends up owning 4 consecutive columns of one row of C and stores them with a
// single 16- or 8-byte write.
#pragma once
#include <type_traits>
#include "gemm_params.hpp"
#include "epilogue.hpp"
#include "gfx950_prims.hpp"

namespace mg {

// Stages one BR x BK operand slice (rows r, k contiguous in LDS).
//   KC  : the stored operand has k contiguous (A with ta=N, B with tb=T);
//         otherwise rows are contiguous and the slice is transposed.
//   VEC : 16-byte global loads are legal (aligned base and ld, and the
//         contiguous extent a multiple of the chunk), else element loads.
template <int ES, int BR, int BK, bool KC, bool VEC, int NT>
struct SliceLoader {
  static constexpr int V = 16 / ES;            // elements per 16-byte chunk
  static constexpr int KCH = BK / V;           // chunks per LDS row
  static constexpr int NCH = BR * KCH;         // chunks per slice
  static constexpr int PITCH = BK * ES;        // LDS row pitch (bytes), unpadded
  static_assert(PITCH == 128, "rows are 8 chunks: the XOR swizzle below assumes it");
  static constexpr int NBLK = KC ? NCH : NCH / V;  // work items (chunk or V x V block)
  static constexpr int ITERS = (NBLK + NT - 1) / NT;
  static constexpr int NREG = KC ? ITERS : ITERS * V;
  static_assert(BK % V == 0 && BR % V == 0, "slice must be whole chunks");

  u32x4 r[NREG];

  // base: byte address of stored element (row r0, k k0) for KC, or of
  // (k k0, row r0) otherwise; ldb: leading dimension in bytes; rv / kv: rows
  // and k values still inside the matrix from this slice's origin.
  __device__ __forceinline__ void load(const char *base, uint32_t ldb, int rv, int kv, int tid) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base);
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int w = tid + it * NT;
      if (NBLK % NT != 0 && w >= NBLK) break;
      if constexpr (KC) {
        const int row = w / KCH, kc = w % KCH;
        if constexpr (VEC) {
          const bool ok = row < rv && kc * V < kv;
          r[it] = buf_load16(rs, ok ? row * ldb + kc * 16 : kOOB);
        } else {
          r[it] = load_elems_k(rs, row, kc, rv, kv, ldb);
        }
      } else {
        const int kb = w % KCH, rb = w / KCH;
        if constexpr (VEC) {
          u32x4 t[V];
#pragma unroll
          for (int j = 0; j < V; ++j) {
            const int k = kb * V + j;
            const bool ok = k < kv && rb * V < rv;
            t[j] = buf_load16(rs, ok ? k * ldb + rb * 16 : kOOB);
          }
          transpose(t, &r[it * V]);
        } else {
#pragma unroll
          for (int i = 0; i < V; ++i) r[it * V + i] = load_elems_r(rs, kb, rb * V + i, rv, kv, ldb);
        }
      }
    }
  }

  __device__ __forceinline__ void store(char *lds, int tid) const {
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int w = tid + it * NT;
      if (NBLK % NT != 0 && w >= NBLK) break;
      if constexpr (KC) {
        const int row = w / KCH, kc = w % KCH;
        *reinterpret_cast<u32x4 *>(lds + row * PITCH + ((kc ^ (row & 7)) * 16)) = r[it];
      } else {
        const int kb = w % KCH, rb = w / KCH;
#pragma unroll
        for (int i = 0; i < V; ++i) {
          const int row = rb * V + i;
          *reinterpret_cast<u32x4 *>(lds + row * PITCH + ((kb ^ (row & 7)) * 16)) = r[it * V + i];
        }
      }
    }
  }

 private:
  // V x V transpose: in[j] holds rows rb*V..+V-1 at k = kb*V + j; out[i]
  // holds k = kb*V..+V-1 of row rb*V + i.
  static __device__ __forceinline__ void transpose(const u32x4 *in, u32x4 *out) {
    if constexpr (ES == 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) out[i] = u32x4{in[0][i], in[1][i], in[2][i], in[3][i]};
    } else {
      // 8 x 8 of 16-bit: element i of in[j] is half (i&1) of dword i/2.
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int d = i >> 1;
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t lo = in[2 * q][d], hi = in[2 * q + 1][d];
          o[q] = (i & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        out[i] = o;
      }
    }
  }

  // Element loads of one chunk: row `row`, k = kc*V .. kc*V+V-1 (KC layout).
  static __device__ __forceinline__ u32x4 load_elems_k(__amdgpu_buffer_rsrc_t rs, int row, int kc,
                                                       int rv, int kv, uint32_t ldb) {
    u32x4 o;
    if constexpr (ES == 4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = kc * 4 + e;
        o[e] = buf_load4(rs, (row < rv && k < kv) ? row * ldb + k * 4 : kOOB);
      }
    } else {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int k = kc * 8 + 2 * d;
        const uint32_t lo = buf_load2(rs, (row < rv && k < kv) ? row * ldb + k * 2 : kOOB);
        const uint32_t hi = buf_load2(rs, (row < rv && k + 1 < kv) ? row * ldb + k * 2 + 2 : kOOB);
        o[d] = lo | (hi << 16);
      }
    }
    return o;
  }

  // Element loads of one chunk from a row-contiguous operand: row `row`,
  // k = kb*V .. kb*V+V-1, stored at k*ld + row.
  static __device__ __forceinline__ u32x4 load_elems_r(__amdgpu_buffer_rsrc_t rs, int kb, int row,
                                                       int rv, int kv, uint32_t ldb) {
    u32x4 o;
    if constexpr (ES == 4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = kb * 4 + e;
        o[e] = buf_load4(rs, (row < rv && k < kv) ? k * ldb + row * 4 : kOOB);
      }
    } else {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int k = kb * 8 + 2 * d;
        const uint32_t lo = buf_load2(rs, (row < rv && k < kv) ? k * ldb + row * 2 : kOOB);
        const uint32_t hi = buf_load2(rs, (row < rv && k + 1 < kv) ? (k + 1) * ldb + row * 2 : kOOB);
        o[d] = lo | (hi << 16);
      }
    }
    return o;
  }
};

template <typename TI, typename TO, int BM_, int BN_, int BK_, int WAVES_M, int WAVES_N, bool A_KC,
          bool B_KC, bool A_VEC, bool B_VEC>
struct GemmTile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int NT = 64 * WAVES_M * WAVES_N;
  static constexpr int ES = sizeof(TI);
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;  // wave sub-tile
  static constexpr int MI = WTM / 16, NJ = WTN / 16;            // 16x16 blocks per wave
  static constexpr int KSTEPS = BK * ES / 64;                   // 4 lane groups x 16 bytes
  using LA = SliceLoader<ES, BM, BK, A_KC, A_VEC, NT>;
  using LB = SliceLoader<ES, BN, BK, B_KC, B_VEC, NT>;
  static constexpr int PITCH = LA::PITCH;
  static constexpr int STAGE_BYTES = (BM + BN) * PITCH;
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be whole MFMA blocks");
  static_assert((BK * ES) % 64 == 0, "BK must be whole k-steps");
  static_assert(2 * STAGE_BYTES <= 160 * 1024, "LDS budget");

  static __device__ __forceinline__ void compute(const char *sa, const char *sb, f32x4 (&acc)[MI][NJ],
                                                 int lane, int wm, int wn) {
    const int lrow = lane & 15;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      // chunk (ks*4 + lane/16) of rows whose index mod 8 is lrow mod 8
      const int col = (((ks * 4 + (lane >> 4)) ^ (lrow & 7)) * 16);
      u32x4 a[MI], b[NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i)
        a[i] = *reinterpret_cast<const u32x4 *>(sa + (wm * WTM + i * 16 + lrow) * PITCH + col);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        b[j] = *reinterpret_cast<const u32x4 *>(sb + (wn * WTN + j * 16 + lrow) * PITCH + col);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) Mfma<TI>::step(acc[i][j], b[j], a[i]);
    }
  }

  static __device__ __forceinline__ void run(const GemmParams &p) {
    __shared__ __attribute__((aligned(16))) char lds[2 * STAGE_BYTES];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    int tm, tn, kb, K;
    work_coords(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, p.splits, p.K, p.k_chunk, tm, tn, kb, K);
    const int m0 = tm * BM, n0 = tn * BN;

    f32x4 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const char *Ab = static_cast<const char *>(p.A);
    const char *Bb = static_cast<const char *>(p.B);
    const uint32_t lda_b = (uint32_t)(p.lda * ES), ldb_b = (uint32_t)(p.ldb * ES);
    const int nk = (K + BK - 1) / BK;

    // Origin of slice kt for each operand (bytes).
    auto a_slice = [&](int kt) -> const char * {
      const int64_t k0 = (int64_t)kb + (int64_t)kt * BK;
      return A_KC ? Ab + ((int64_t)m0 * p.lda + k0) * ES : Ab + (k0 * p.lda + m0) * ES;
    };
    auto b_slice = [&](int kt) -> const char * {
      const int64_t k0 = (int64_t)kb + (int64_t)kt * BK;
      return B_KC ? Bb + ((int64_t)n0 * p.ldb + k0) * ES : Bb + (k0 * p.ldb + n0) * ES;
    };

    LA la;
    LB lb;
    if (nk > 0) {
      la.load(a_slice(0), lda_b, p.M - m0, K, tid);
      lb.load(b_slice(0), ldb_b, p.N - n0, K, tid);
      la.store(lds, tid);
      lb.store(lds + BM * PITCH, tid);
    }
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
      char *cur = lds + (kt & 1) * STAGE_BYTES;
      char *nxt = lds + ((kt + 1) & 1) * STAGE_BYTES;
      const bool more = kt + 1 < nk;
      if (more) {
        const int kv = K - (kt + 1) * BK;
        la.load(a_slice(kt + 1), lda_b, p.M - m0, kv, tid);
        lb.load(b_slice(kt + 1), ldb_b, p.N - n0, kv, tid);
      }
      compute(cur, cur + BM * PITCH, acc, lane, wm, wn);
      if (more) {
        la.store(nxt, tid);
        lb.store(nxt + BM * PITCH, tid);
      }
      __syncthreads();
    }

    if (p.splits > 1)
      GemmEpilogue<float, MI, NJ>::store(partial_params(p, kb), acc, m0 + wm * WTM, n0 + wn * WTN, lane);
    else
      GemmEpilogue<TO, MI, NJ>::store(p, acc, m0 + wm * WTM, n0 + wn * WTN, lane);
  }

};

template <class Tile>
__global__ void __launch_bounds__(Tile::NT) gemm_kernel(GemmParams p) {
  Tile::run(p);
}

// C = beta * C (alpha == 0 or K == 0): A and B are not read; beta == 0
// writes zeros without reading C.
template <typename TO>
__global__ void __launch_bounds__(256) scale_c_kernel(GemmParams p) {
  TO *C = static_cast<TO *>(p.C);
  const int64_t total = (int64_t)p.M * p.N;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = idx / p.N, n = idx - m * p.N;
    TO *c = C + m * p.ldc + n;
    // alpha * (empty or ignored product) contributes +0: 0 + beta*C (so a
    // -0 product beta*C becomes +0, as in the formula's left-to-right sum).
    *c = from_f32<TO>(p.beta == 0.0f ? 0.0f : 0.0f + p.beta * to_f32(*c));
  }
}

// Operand repack: rows x cols elements of ES bytes at src (row pitch ld
// elements) copied to dst with row pitch `pitch` (a multiple of 16 bytes),
// columns cols .. pitch-1 zero.  The copy is 16-byte loadable, and the
// zeros make a chunk that straddles the last column safe to read.
template <int ES>
__global__ void __launch_bounds__(256) pack_rows_kernel(const void *src, int64_t ld, int64_t rows,
                                                        int64_t cols, void *dst, int64_t pitch) {
  typedef typename std::conditional<ES == 4, uint32_t, uint16_t>::type T;
  const T *s = static_cast<const T *>(src);
  T *d = static_cast<T *>(dst);
  const int64_t total = rows * pitch;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / pitch, c = i - r * pitch;
    d[i] = c < cols ? s[r * ld + c] : (T)0;
  }
}

// Stream-K arrival counters to zero before the tile kernel (a kernel, not a
// memset, so the call can be captured in a HIP graph).
template <int Unused = 0>
__global__ void __launch_bounds__(256) zero_ints_kernel(int *p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

// Split-K reduction: C = alpha * (P_0 + P_1 + ... + P_{S-1}) + beta * C with
// the partials summed in split order, so the result does not depend on
// which split finished first; one rounding to the C type, and beta == 0
// never reads C.  Each thread owns 4 consecutive columns of one row.
template <typename TO>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(GemmParams p) {
  const int64_t slab = (int64_t)p.M * p.N;
  const int ng = (p.N + 3) / 4;
  const int64_t total = (int64_t)p.M * ng;
  const bool use_beta = p.beta != 0.0f;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
       g += (int64_t)gridDim.x * blockDim.x) {
    const int m = (int)(g / ng), n = (int)(g - (int64_t)m * ng) * 4;
    const float *w = p.ws + (int64_t)m * p.N + n;
    float x[4] = {0.f, 0.f, 0.f, 0.f};
    if ((p.N & 3) == 0) {
      for (int s = 0; s < p.splits; ++s) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(w + s * slab);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] += v[e];
      }
    } else {
      for (int s = 0; s < p.splits; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < p.N) x[e] += w[s * slab + e];
    }
    if (p.row_exp != nullptr) GemmEpilogue<TO, 1, 1>::unscale(p, m, n, x);
    GemmEpilogue<TO, 1, 1>::store4(p, static_cast<TO *>(p.C) + (int64_t)m * p.ldc, n, x, use_beta);
  }
}

}  // namespace mg
