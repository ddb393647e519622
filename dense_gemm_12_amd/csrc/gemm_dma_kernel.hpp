// 16-bit-input GEMM built around gfx950's global->LDS DMA, for every storage
// layout of A and B:
//
//   * buffer_load_dwordx4 ... lds moves each 16-byte chunk from HBM straight
//     into LDS without passing through VGPRs, so no staging registers and no
//     ds_write instructions are spent on the copy;
//   * one DMA instruction writes 64 lanes x 16 bytes = 1 KiB of LDS at
//     consecutive addresses, so rows cannot be padded; bank conflicts on the
//     fragment reads are avoided instead by XOR-permuting the 16-byte chunks
//     within each LDS row (the idea "HGEMM SMEM Swizzle 代码学习" applies to
//     ldmatrix; the permutations here were chosen by measuring gfx950's LDS
//     conflict counters).  The DMA side applies the same permutation when it
//     picks which global chunk each lane fetches;
//   * an operand whose k dimension is contiguous in memory (A stored M x K, B
//     stored N x K: the "TN" layout of "HGEMM SMEM Swizzle 代码学习" and of "Warp
//     Specialization HGEMM" section 6) is staged as [row][k] and read with one
//     ds_read_b128 per 16x32 fragment; a k-major operand (A stored K x M, B
//     stored K x N as in the plain row-major problem of "SGEMM CUDA代码学习") is
//     staged untouched as [k][row] and read with two ds_read_b64_tr_b16, the
//     gfx950 LDS read that transposes 16-bit elements across each group of 16
//     lanes, so no layout ever needs a transpose pass or register shuffles;
//   * STAGES slices ring through LDS and each wave reads the fragments of the
//     next k-step while the MFMAs of the current one run ("SGEMM CUDA代码学习"
//     steps 4-5 and the worklog's closing notes on two-level buffering,
//     restated for vmcnt-counted DMA); the issue order of MFMAs, LDS reads
//     and DMA is fixed with scheduling fences.
// Tails: rows past M/N and k past K are fetched with an out-of-range buffer
// offset, which makes the DMA write zeros; slices beyond the last one are
// issued the same way so the vmcnt bookkeeping never changes.
#pragma once
#include "epilogue.hpp"
#include "gemm_params.hpp"
#include "gfx950_prims.hpp"

namespace mg {

typedef __attribute__((address_space(3))) void lds_void;
typedef short i16x4 __attribute__((ext_vector_type(4)));

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14
  __builtin_amdgcn_s_waitcnt((N & 0xf) | (0x7 << 4) | (0xf << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// ds_read_b64_tr_b16 as inline assembly.  The compiler's builtin for it is
// treated as possibly reading what any LDS DMA still in flight writes, so a
// vmcnt(0) wait goes in front of it, which drains every slice of DMA the
// schedules keep in flight.  The schedules order these reads against the
// DMA themselves (vmcnt waits and barriers), and since the compiler does
// not know the result arrives later, they also wait for it explicitly
// (lgkmcnt(0) followed by a scheduling fence, so that no MFMA is moved
// above the wait) before any MFMA reads it.
__device__ __forceinline__ u32x2 ds_read_tr16_b64(const char *p) {
  const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
  u32x2 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(a));
  return v;
}

// Waits for this wave's LDS reads and keeps every later instruction below.
__device__ __forceinline__ void wait_lgkm0_fenced() {
  __builtin_amdgcn_sched_barrier(0);
  wait_lgkm0();
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier for LDS hand-offs whose completion the caller has
// already established with explicit vmcnt/lgkmcnt waits.  Unlike
// __syncthreads() it carries no memory fence, so DMA issued for later slices
// stays in flight across it; the empty asm statements keep the compiler from
// moving LDS accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// One operand slice (R rows of the operand x BK values of k, ES-byte
// elements) in LDS.  V = 16 / ES elements make one 16-byte chunk; a "k-step"
// is the 64 bytes of k that the four 16-lane groups of a wave cover with one
// chunk each (32 k of 16-bit data, 16 k of fp32).
//
// KC = true, k contiguous in memory: LDS rows are operand rows of BK*ES
// bytes; 16-byte chunk c of row r sits at slot c ^ swz(r), swz(r) = r mod 8
// (128-byte rows) or (r / 2) mod 4 (64-byte rows).  Lane l's fragment for
// 16-row block b, k-step ks is row 16b + l%16, chunk 4ks + l/16: one
// ds_read_b128 (for fp32 its four floats are the four k sub-steps
// 4(l/16) + s of the k-step).
//
// KC = false, operand rows contiguous in memory: LDS rows are the BK k
// values, each R*ES bytes.
//   16-bit: chunk c of k-row k sits at slot c ^ swz(k), swz(k) = 2 * ((k mod
//   4) | ((k / 8) mod 2) * 4), an even value so the two 16-byte chunks of
//   each 32-byte span stay adjacent.  ds_read_b64_tr_b16 returns to lane j of
//   a 16-lane group element j%4 of the 8-byte reads of lanes j/4, j/4+4,
//   j/4+8, j/4+12 of the group; so lane i of group g reads k-row 8g + 4h +
//   i/4 at columns 16b + 4(i%4) .. +3 and receives, for its own column 16b +
//   j, the four k values 8g + 4h .. +3.  Two reads (h = 0, 1) give the 8 k
//   values of the MFMA operand.
//   fp32: no permutation.  Read number r = 4q + s of a k-step has lane j of
//   group g load k-row 16ks + 4g + s at operand rows 64q + 4j .. +3 (one
//   aligned 256-byte span per 16-lane group, so conflict-free); float t of it
//   is the sub-step-s value of 16-row block 4q + t, whose lane-j row is
//   64q + 4j + t.  The tile therefore orders the rows of each 64-row quad as
//   (4j + t), and the epilogue maps them back.
// Whether DmaOperand<R, BK, KC, NW, ES> has a supported LDS layout: whole
// 1 KiB DMA blocks per wave; k-contiguous rows of 64 or 128 bytes, or k-major
// rows of at least 256 bytes that tile a 1 KiB block.
template <int R, int BK, bool KC, int NW, int ES>
constexpr bool dma_operand_ok() {
  const int bytes = R * BK * ES, rowb = KC ? BK * ES : R * ES, cpr = rowb / 16;
  return bytes % (1024 * NW) == 0 && (KC ? (cpr == 4 || cpr == 8) : (cpr >= 16 && 1024 % rowb == 0));
}

template <int R, int BK, bool KC, int NW, int ES = 2>
struct DmaOperand {
  static constexpr int V = 16 / ES;
  static constexpr int BYTES = R * BK * ES;
  static constexpr int INST = BYTES / 1024 / NW;  // DMA instructions per wave per slice
  static constexpr int ROWB = KC ? BK * ES : R * ES;
  static constexpr int CPR = ROWB / 16;
  static constexpr int RPB = 1024 / ROWB;         // LDS rows per 1 KiB DMA block
  static constexpr int READS = (KC || ES == 4) ? 1 : 2;  // LDS reads per fragment register
  static constexpr int KSTEP = 64 / ES;           // k values per k-step
  static_assert(ES == 2 || ES == 4, "16-bit or fp32 elements");
  static_assert(BYTES % (1024 * NW) == 0, "whole DMA blocks per wave");
  static_assert(KC ? (CPR == 4 || CPR == 8) : (CPR >= 16 && 1024 % ROWB == 0),
                "supported LDS row widths");

  static __device__ __forceinline__ int swz(int row) {
    if constexpr (KC) return CPR == 8 ? (row & 7) : ((row >> 1) & 3);
    else if constexpr (ES == 2) return 2 * ((row & 3) | (((row >> 3) & 1) << 2));
    else return 0;
  }

  // DMA instruction u of this wave for one slice.  rs: buffer at the stored
  // element (r0, k0) (KC) or (k0, r0) (k-major); ldb: row pitch in bytes;
  // rv / kv: operand rows and k values still inside the matrix.
  static __device__ __forceinline__ void dma(__amdgpu_buffer_rsrc_t rs, uint32_t ldb, int rv, int kv,
                                             char *dst, int wave, int lane, int u) {
    const int blk = wave * INST + u;
    const int row = blk * RPB + lane / CPR;
    const int c = (lane % CPR) ^ swz(row);
    const bool ok = KC ? (row < rv && c * V < kv) : (row < kv && c * V < rv);
    const uint32_t off = ok ? row * ldb + c * 16 : kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(dst + blk * 1024), 16, off, 0, 0, 0);
  }

  // Per-lane fragment addressing.  rowblk0: first 16-row block of the wave
  // within the slice; NB: fragment registers per k-step (16-row blocks; for
  // fp32 k-major, reads 4q + s); KSTEPS: k-steps per slice.
  template <int NB, int KSTEPS>
  struct Frag {
    static constexpr bool TR16 = !KC && ES == 2;
    int base;
    int xo[KC ? KSTEPS : (TR16 ? NB : 1)];

    __device__ __forceinline__ void init(int lane, int rowblk0) {
      const int j = lane & 15, g = lane >> 4;
      if constexpr (KC) {
        base = (rowblk0 * 16 + j) * ROWB;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) xo[ks] = ((ks * 4 + g) ^ swz(j)) * 16;
      } else if constexpr (TR16) {
        const int gk = 2 * ((j >> 2) | ((g & 1) << 2));  // swz of the lane's k-row
        base = (8 * g + (j >> 2)) * ROWB + 8 * (j & 1);
#pragma unroll
        for (int b = 0; b < NB; ++b) xo[b] = ((((rowblk0 + b) * 2) ^ gk) + ((j >> 1) & 1)) * 16;
      } else {
        static_assert(KC || TR16 || NB % 4 == 0, "fp32 k-major fragments come in 64-row quads");
        base = 4 * g * ROWB + rowblk0 * 16 * ES + 16 * j;
        xo[0] = 0;
      }
    }

    // Read number h (0 .. READS-1) of fragment register b, k-step ks, into f.
    __device__ __forceinline__ void read(const char *st, int b, int ks, int h, u32x4 &f) const {
      if constexpr (KC) {
        f = *reinterpret_cast<const u32x4 *>(st + base + b * 16 * ROWB + xo[ks]);
      } else if constexpr (TR16) {
        const u32x2 w = ds_read_tr16_b64(st + base + (ks * 32 + 4 * h) * ROWB + xo[b]);
        if (h == 0) {
          f.x = w.x;
          f.y = w.y;
        } else {
          f.z = w.x;
          f.w = w.y;
        }
      } else {
        f = *reinterpret_cast<const u32x4 *>(st + base + (ks * KSTEP + (b & 3)) * ROWB + (b >> 2) * 256);
      }
    }
  };
};

template <typename TI, typename TO, int BM_, int BN_, int BK_, int STAGES_, int WAVES_M, int WAVES_N,
          bool A_KC, bool B_KC, bool PINGPONG = false, bool STREAMK = false>
struct DmaTile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_;
  static constexpr int NW = WAVES_M * WAVES_N, NT = 64 * NW;
  static constexpr int ES = sizeof(TI);
  using OA = DmaOperand<BM, BK, A_KC, NW, ES>;
  using OB = DmaOperand<BN, BK, B_KC, NW, ES>;
  static constexpr int A_BYTES = OA::BYTES, B_BYTES = OB::BYTES;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int A_INST = OA::INST, B_INST = OB::INST;
  static constexpr int LOADS_PER_SLICE = A_INST + B_INST;
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  static constexpr int MI = WTM / 16, NJ = WTN / 16;
  static constexpr int KSTEPS = BK * ES / 64;      // k-steps (64 bytes of k) per slice
  static constexpr int RD_B = NJ * OB::READS, RD_A = MI * OA::READS;
  // MFMA instructions per k-step: one 16x16x32 per block pair for 16-bit
  // inputs, four 16x16x4 (sub-steps s) for fp32.
  static constexpr int SUB = Mfma<TI>::kInsts;
  static constexpr int MFMAS = MI * NJ * SUB;
  // fp32 k-major operands order the rows of each 64-row quad as 4j + t.
  static constexpr bool A_Q = ES == 4 && !A_KC, B_Q = ES == 4 && !B_KC;
  // k-major 16-bit fragments come from ds_read_tr16_b64, whose results the
  // schedules wait for explicitly.
  static constexpr bool ASM_READS = ES == 2 && (!A_KC || !B_KC);
  static_assert(KSTEPS == 1 || KSTEPS == 2, "one or two k-steps per slice");
  static_assert(STAGES * STAGE_BYTES <= 160 * 1024, "LDS budget");
  static_assert(LOADS_PER_SLICE * (STAGES - 1) < 64, "vmcnt range");

  // LDS: the slice ring, and for stream-K one more word (the "last
  // contributor" flag) in the same array.  A second __shared__ object makes
  // the compiler put a vmcnt(0) wait in front of ring reads that it can no
  // longer tell apart from the DMA in flight.
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES + (STREAMK ? 16 : 0);

  static __device__ __forceinline__ void run(const GemmParams &p) {
    __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    f32x4 acc[MI][NJ];
    if constexpr (STREAMK) {
      stream_k(p, lds, wave, lane, wm, wn, acc);
    } else {
      int tm, tn, kb, K;
      work_coords(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, p.splits, p.K, p.k_chunk, tm, tn, kb, K);
      const int m0 = tm * BM, n0 = tn * BN;
      compute(p, lds, m0, n0, kb, K, wave, lane, wm, wn, acc);
      if (p.splits > 1)
        GemmEpilogue<float, MI, NJ, A_Q, B_Q>::store(partial_params(p, kb), acc, m0 + wm * WTM,
                                                     n0 + wn * WTN, lane);
      else
        GemmEpilogue<TO, MI, NJ, A_Q, B_Q>::store(p, acc, m0 + wm * WTM, n0 + wn * WTN, lane);
    }
  }

  // Stream-K schedule ("Stream-K: Work-centric Parallel Decomposition for
  // Dense Matrix-Matrix Multiplication on the GPU", Osama, Merrill, Cecka,
  // Garland and Owens, 2023), the persistent form of the split-K idea the
  // worklog's Kernel 10 section sees cuBLAS use: the grid is p.sk_grid
  // workgroups of one round of the chip, after p.sk_dp_tiles workgroups
  // that each take one whole tile in the plain grid's order (all rounds but
  // the last one or two: these are dispatched first, and the hardware
  // balances them over the CUs as in the plain grid).  The slice iterations
  // of the remaining tiles are cut into p.sk_grid equal contiguous ranges,
  // and each of the last p.sk_grid workgroups runs its range tile by tile.
  // A tile covered whole by one
  // workgroup is finished there; a tile whose slices are shared by several
  // workgroups ("contributors", ordered by k) is finished by the one that
  // completes last, with no waiting:
  //   every contributor stores its fp32 sums to its own workspace slot (2w
  //   for the tile its range starts in, 2w + 1 for the tile it ends in, in
  //   the accumulator register layout, 1 KiB per store instruction) with
  //   device-coherent stores, waits until they are acknowledged and
  //   increments the tile's counter; the contributor that sees the count
  //   reach the number of contributors reads every slot back with
  //   device-coherent loads, adds them in contributor order (so the result
  //   does not depend on which one finished last) and runs the alpha/beta
  //   epilogue.
  // Ranges of different workgroups end at different points of their tiles,
  // so epilogues are spread over the run instead of coming in one burst per
  // round, and no round is left partly empty.  The counters (p.sk_cnt, one
  // per tile) must be zero at launch; tiles x sk_ipt < 2^31 (host-checked).
  static __device__ __forceinline__ int sk_start(const GemmParams &p, int total, int w) {
    return (int)((int64_t)total * w / p.sk_grid);
  }
  static __device__ __forceinline__ int sk_owner(const GemmParams &p, int total, int it) {
    int w = (int)((int64_t)it * p.sk_grid / total);  // start(w) <= it up to rounding; step to the exact owner
    while (w + 1 < p.sk_grid && sk_start(p, total, w + 1) <= it) ++w;
    while (w > 0 && sk_start(p, total, w) > it) --w;
    return w;
  }

  static __device__ __forceinline__ void stream_k(const GemmParams &p, char *lds, int wave, int lane, int wm,
                                                  int wn, f32x4 (&acc)[MI][NJ]) {
    int &s_last = *reinterpret_cast<int *>(lds + STAGES * STAGE_BYTES);
    const int ipt = p.sk_ipt, G = p.sk_grid;
    const int dp = p.sk_dp_tiles;  // leading whole tiles, one workgroup each, dispatched first
    const int total = (p.tiles_m * p.tiles_n - dp) * ipt;  // slice iterations of the stream-K tail
    const int b = blockIdx.x;
    // tail workgroups: logical index w, each XCD gets a contiguous block of ranges
    const int w = b < dp ? 0 : remap_xcd(b - dp, G);
    int it = b < dp ? 0 : sk_start(p, total, w);
    const int it1 = b < dp ? 0 : sk_start(p, total, w + 1);
    constexpr int TILE_F4 = BM * BN / 4;  // f32x4 per partial slot
    for (bool whole = b < dp; whole || it < it1;) {
      int t, kbeg, kend;
      if (whole) {  // a data-parallel workgroup: one tile, whole, in the plain grid's order
        t = remap_xcd(b, dp);
        kbeg = 0;
        kend = ipt;
        whole = false;
      } else {  // the stream-K tail: this workgroup's slice range, tile by tile
        const int tt = it / ipt;
        kbeg = it - tt * ipt;
        kend = min(ipt, kbeg + (it1 - it));
        t = dp + tt;
        it += kend - kbeg;
      }
      // Per-lane values are recomputed in every unit: made opaque here, they
      // are not hoisted out of this loop to stay live (and spill) across the
      // whole k-loop.
      int ln = lane;
      asm volatile("" : "+v"(ln));
      int tm, tn;
      tile_coords(t, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
      const int m0 = tm * BM, n0 = tn * BN;
      const int kb = kbeg * BK;
      __syncthreads();  // every wave is done with the previous unit's LDS before the ring refills
      compute(p, lds, m0, n0, kb, min(p.K - kb, (kend - kbeg) * BK), wave, ln, wm, wn, acc);
      if (kbeg != 0 || kend != ipt) {
        const int tt = t - dp;
        const int wf = sk_owner(p, total, tt * ipt);
        const int nc = sk_owner(p, total, (tt + 1) * ipt - 1) - wf + 1;  // contributors
        // Partial sums move with device-scope buffer accesses (cache policy
        // SC1): a store is acknowledged once it is coherent for every XCD,
        // and a load is served coherently, bypassing stale copies in this
        // CU's L1 and this XCD's L2.  So no L2-wide write-back or invalidate
        // (the agent-scope fences) is needed, which would also throw away
        // the operand tiles the XCD's other workgroups are reading.
        constexpr int kDeviceScope = 16;  // SC1
        const __amdgpu_buffer_rsrc_t ws = make_rsrc(p.ws);
        // byte offset of this lane's f32x4 of accumulator block (i, j) in the
        // slot of contributor v for tile t: 2v if tile t is where v's range
        // starts, else 2v + 1
        const uint32_t lane_off = (uint32_t)(wave * MI * NJ * 64 + ln) * 16;
        auto slot = [&](int v) -> uint32_t {
          const int first = sk_start(p, total, v) / ipt == tt ? 0 : 1;
          return (uint32_t)(2 * v + first) * (TILE_F4 * 16) + lane_off;
        };
        {
          const uint32_t mine = slot(w);
#pragma unroll
          for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][j]), ws,
                                                     mine + (i * NJ + j) * 1024, 0, kDeviceScope);
        }
        wait_vmcnt<0>();  // this wave's sums are coherent device-wide
        __syncthreads();
        if (threadIdx.x == 0) {
          const int old = __hip_atomic_fetch_add(p.sk_cnt + t, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          s_last = old == nc - 1;
        }
        __syncthreads();
        if (!s_last) continue;
        // The last contributor: every slot, its own included, in contributor order.
        {
          const uint32_t first = slot(wf);
#pragma unroll
          for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
              acc[i][j] = __builtin_bit_cast(
                  f32x4, __builtin_amdgcn_raw_buffer_load_b128(ws, first + (i * NJ + j) * 1024, 0, kDeviceScope));
        }
        for (int q = 1; q < nc; ++q) {
          const uint32_t sq = slot(wf + q);
#pragma unroll
          for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
              acc[i][j] += __builtin_bit_cast(
                  f32x4, __builtin_amdgcn_raw_buffer_load_b128(ws, sq + (i * NJ + j) * 1024, 0, kDeviceScope));
        }
      }
      GemmEpilogue<TO, MI, NJ, A_Q, B_Q, false>::store(p, acc, m0 + wm * WTM, n0 + wn * WTN, ln);
    }
  }

  // The k-loop of one work unit: the tile at (m0, n0), k in [kb, kb + K).
  // Leaves the unit's sums in acc; on return every DMA and LDS read of the
  // unit has completed (the LDS ring may be refilled after a barrier).
  static __device__ __forceinline__ void compute(const GemmParams &p, char *lds, int m0, int n0, int kb, int K,
                                                 int wave, int lane, int wm, int wn, f32x4 (&acc)[MI][NJ]) {
    // Slice origins advance by BK along k: BK elements for a k-contiguous
    // operand, BK rows for a k-major one.
    const char *Ab = static_cast<const char *>(p.A) +
                     (A_KC ? (int64_t)m0 * p.lda + kb : (int64_t)kb * p.lda + m0) * ES;
    const char *Bb = static_cast<const char *>(p.B) +
                     (B_KC ? (int64_t)n0 * p.ldb + kb : (int64_t)kb * p.ldb + n0) * ES;
    const int64_t a_step = (A_KC ? BK : (int64_t)BK * p.lda) * ES;
    const int64_t b_step = (B_KC ? BK : (int64_t)BK * p.ldb) * ES;
    const uint32_t lda_b = (uint32_t)(p.lda * ES), ldb_b = (uint32_t)(p.ldb * ES);
    const int rva = p.M - m0, rvb = p.N - n0;
    const int nk = (K + BK - 1) / BK;

    auto dma_op = [&](int kt, int u) {  // DMA instruction u (A first, then B) of slice kt
      char *st = lds + (kt % STAGES) * STAGE_BYTES;
      const int kv = K - kt * BK;
      if (u < A_INST)
        OA::dma(make_rsrc(Ab + kt * a_step), lda_b, rva, kv, st, wave, lane, u);
      else
        OB::dma(make_rsrc(Bb + kt * b_step), ldb_b, rvb, kv, st + A_BYTES, wave, lane, u - A_INST);
    };
    auto issue = [&](int kt) {
#pragma unroll
      for (int u = 0; u < LOADS_PER_SLICE; ++u) dma_op(kt, u);
    };

#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    typename OA::template Frag<MI, KSTEPS> fra;
    typename OB::template Frag<NJ, KSTEPS> frb;
    fra.init(lane, wm * MI);
    frb.init(lane, wn * NJ);

    // Memory op t of a fragment set: B-side reads first, then A-side.
    auto read_op = [&](const char *st, int ks, int t, u32x4 (&fa)[MI], u32x4 (&fb)[NJ]) {
      if (t < RD_B) frb.read(st + A_BYTES, t / OB::READS, ks, t % OB::READS, fb[t / OB::READS]);
      else fra.read(st, (t - RD_B) / OA::READS, ks, (t - RD_B) % OA::READS, fa[(t - RD_B) / OA::READS]);
    };
    auto read_frags = [&](const char *st, int ks, u32x4 (&fa)[MI], u32x4 (&fb)[NJ]) {
#pragma unroll
      for (int t = 0; t < RD_A + RD_B; ++t) read_op(st, ks, t, fa, fb);
    };
    // MFMA instruction t of a k-step, sub-step-major so that consecutive
    // instructions never share an accumulator.
    auto mfma = [&](int t, const u32x4 (&fa)[MI], const u32x4 (&fb)[NJ]) {
      const int s = t / (MI * NJ), i = (t % (MI * NJ)) / NJ, j = t % NJ;
      if constexpr (SUB == 1) {
        Mfma<TI>::step(acc[i][j], fb[j], fa[i]);
      } else {
        const float a = __builtin_bit_cast(float, A_Q ? fa[(i & ~3) + s][i & 3] : fa[i][s]);
        const float b = __builtin_bit_cast(float, B_Q ? fb[(j & ~3) + s][j & 3] : fb[j][s]);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(b, a, acc[i][j], 0, 0, 0);
      }
    };
    auto mfmas = [&](const u32x4 (&fa)[MI], const u32x4 (&fb)[NJ]) {
#pragma unroll
      for (int t = 0; t < MFMAS; ++t) mfma(t, fa, fb);
    };

    if constexpr (PINGPONG) {
      // Ping-pong schedule, gfx950's form of the pages' producer/consumer
      // split ("Warp Specialization HGEMM": copy warps feed compute warps
      // through a ring).  The eight waves form two groups of four, one wave
      // of each group per SIMD (waves w and w + 4 share SIMD w), and every
      // wave alternates between a memory phase and a compute phase:
      //   memory phase of slice i: issue this wave's share of the DMA for
      //     slice i + STAGES - 1 (into the buffer of slice i - 1), then read
      //     its slice-i fragments from LDS into registers;
      //   compute phase of slice i: the slice's MFMAs, nothing else.
      // Group 1 starts one phase late, so on each SIMD one wave issues MFMAs
      // back to back while its partner issues the memory instructions, and
      // no MFMA waits behind a DMA that cannot issue yet.  A barrier ends
      // every phase (each wave first waits until all but its STAGES - 2
      // newest slices of DMA have landed):
      //   - slice i is read by group 0 in phase 2i and by group 1 in phase
      //     2i + 1, so its buffer is free from phase 2i + 2 on, when the
      //     memory phase of slice i + 1 refills it;
      //   - a wave's share of slice i + STAGES - 1 goes out in phase 2i or
      //     2i + 1 and is read from phase 2i + 2 STAGES - 2 on.
      // Both groups pass 2 nk barriers (group 1's first phase is idle and its
      // last compute phase ends without one), so the counts match for any nk.
      // A wave's fragment registers are rewritten by its next memory phase
      // only after the phase barrier and the DMA issue (some thirty
      // instructions), far past the operand reads of its last MFMA.
      static_assert(NW == 8 && KSTEPS == 1 && STAGES >= 3, "ping-pong: 8 waves, one-k-step slices, >= 3 stages");
      const int grp = wave >> 2;
      u32x4 fa[MI], fb[NJ];
#pragma unroll
      for (int s = 0; s < STAGES - 1; ++s) issue(s);
      wait_vmcnt<LOADS_PER_SLICE * (STAGES - 2)>();
      lds_barrier();
      auto memory_phase = [&](int i) {
#pragma unroll
        for (int u = 0; u < LOADS_PER_SLICE; ++u) dma_op(i + STAGES - 1, u);
        read_frags(lds + (i % STAGES) * STAGE_BYTES, 0, fa, fb);
        wait_lgkm0();
      };
      auto end_phase = [&]() {
        __builtin_amdgcn_sched_barrier(0);  // the phase's MFMAs stay before its barrier
        wait_vmcnt<LOADS_PER_SLICE * (STAGES - 2)>();
        lds_barrier();
      };
      if (grp == 0) {
        for (int i = 0; i < nk; ++i) {
          memory_phase(i);
          end_phase();
          mfmas(fa, fb);
          end_phase();
        }
      } else {
        if (nk > 0) end_phase();  // (nk is uniform: with no slices neither group passes a barrier)
        for (int i = 0; i < nk; ++i) {
          memory_phase(i);
          end_phase();
          mfmas(fa, fb);
          if (i + 1 < nk) end_phase();
        }
      }
    } else if constexpr (KSTEPS == 2) {
      // Mid-slice barrier schedule.  Per slice kt (buffer S = kt % STAGES):
      //   phase A: MFMAs of k-step 0, each followed by at most one LDS read
      //            of the k-step 1 fragments of slice kt;
      //   wait for slice kt+1's DMA (slices kt+2 .. kt+STAGES-1 stay in
      //   flight) and for this wave's reads; barrier: every wave now holds
      //   all of slice kt's fragments, so buffer S is free;
      //   phase C: MFMAs of k-step 1, each followed by LDS reads of slice
      //            kt+1's k-step 0 fragments, and every DSTR-th one also by
      //            one DMA issue for slice kt+STAGES (into S).  Issued back to
      //            back, a wave's DMA filled the texture unit's command queue
      //            and stalled its MFMAs behind it.
      // (With more reads than MFMAs, each MFMA is followed by up to
      // ceil(reads / MFMAs) of them.)  The MFMAs never wait on an LDS read; the
      // barrier is the only point where the matrix pipe can drain.  With two
      // stages a slice's DMA has one slice of time to land; every further
      // stage adds one (the 4-wave 128 x 128 tiles, one workgroup per CU,
      // need the second).
      constexpr int SLOTS = MFMAS;
      constexpr int PA = (RD_A + RD_B + SLOTS - 1) / SLOTS;                    // ops per MFMA, phase A
      // phase C: the next k-step's reads first (PCR after each MFMA), and the
      // slice's DMA spread evenly, one after every DSTR-th MFMA
      constexpr int PCR = (RD_A + RD_B + SLOTS - 1) / SLOTS;
      static_assert(LOADS_PER_SLICE <= SLOTS, "one DMA issue per MFMA at most");
      constexpr int DSTR = SLOTS / LOADS_PER_SLICE;
      // With two waves per SIMD, a wave in phase C (which carries the
      // slice's DMA) issues ahead of a partner that has already moved on to
      // phase A of the next slice (wave priority, s_setprio), so the DMA goes
      // out sooner and the pair reaches the next barrier closer together.
      constexpr bool PRIO = NW >= 8;
      u32x4 fa0[MI], fb0[NJ], fa1[MI], fb1[NJ];
#pragma unroll
      for (int s = 0; s < STAGES; ++s) issue(s);
      wait_vmcnt<LOADS_PER_SLICE * (STAGES - 1)>();  // slice 0 landed; the rest stay in flight
      lds_barrier();
      read_frags(lds, 0, fa0, fb0);
      for (int kt = 0; kt < nk; ++kt) {
        const char *st = lds + (kt % STAGES) * STAGE_BYTES;
        const char *nx = lds + ((kt + 1) % STAGES) * STAGE_BYTES;
        if constexpr (ASM_READS) wait_lgkm0_fenced();  // fa0 / fb0 (prologue or last phase C)
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int t = 0; t < SLOTS; ++t) {  // phase A
          mfma(t, fa0, fb0);
#pragma unroll
          for (int o = t * PA; o < (t + 1) * PA; ++o)
            if (o < RD_A + RD_B) read_op(st, 1, o, fa1, fb1);
          __builtin_amdgcn_sched_barrier(0);
        }
        wait_vmcnt<LOADS_PER_SLICE * (STAGES - 2)>();  // slice kt+1 landed
        wait_lgkm0_fenced();  // this wave's reads of S are done (phase C's fragments included)
        lds_barrier();
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int t = 0; t < SLOTS; ++t) {  // phase C
          mfma(t, fa1, fb1);
#pragma unroll
          for (int o = t * PCR; o < (t + 1) * PCR; ++o)
            if (o < RD_A + RD_B) read_op(nx, 0, o, fa0, fb0);
          if (t % DSTR == 0 && t / DSTR < LOADS_PER_SLICE) dma_op(kt + STAGES, t / DSTR);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
    } else if constexpr (STAGES >= 3 && KSTEPS == 1) {
      // Ring schedule for one-k-step slices.  During slice kt each wave runs
      // its MFMAs on slice kt's fragments (in registers), interleaved with
      // the LDS reads of slice kt+1's fragments and the DMA of slice
      // kt+STAGES into buffer kt % STAGES (free: slice kt's fragments were
      // read by every wave before the previous barrier).  The barrier at the
      // end of slice kt waits only for slice kt+2, so STAGES-1 slices of DMA
      // stay in flight.
      constexpr int SLOTS = MFMAS;
      constexpr int PO = (LOADS_PER_SLICE + RD_A + RD_B + SLOTS - 1) / SLOTS;  // ops per MFMA
      u32x4 fa[2][MI], fb[2][NJ];
#pragma unroll
      for (int s = 0; s < STAGES; ++s) issue(s);
      wait_vmcnt<LOADS_PER_SLICE * (STAGES - 2)>();
      lds_barrier();
      read_frags(lds, 0, fa[0], fb[0]);
      // Slice 0's buffer is refilled during slice 0: every wave must have
      // its slice-0 fragments before anyone issues that DMA.
      wait_lgkm0();
      lds_barrier();
      for (int kt = 0; kt < nk; kt += 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {  // two slices per trip keep fragment buffers static
          const int k = kt + h;
          const char *nx = lds + ((k + 1) % STAGES) * STAGE_BYTES;
#pragma unroll
          for (int t = 0; t < SLOTS; ++t) {
            mfma(t, fa[h], fb[h]);
#pragma unroll
            for (int o = t * PO; o < (t + 1) * PO; ++o) {
              if (o < RD_A + RD_B) read_op(nx, 0, o, fa[h ^ 1], fb[h ^ 1]);
              else if (o < RD_A + RD_B + LOADS_PER_SLICE) dma_op(k + STAGES, o - RD_A - RD_B);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          if (k + 1 >= nk) break;
          wait_vmcnt<LOADS_PER_SLICE * (STAGES - 2)>();  // slice k+2 has landed
          wait_lgkm0();                                   // slice k+1's reads are done
          lds_barrier();
        }
      }
    } else {
      // Plain loop for one-k-step slices in two stages: one barrier per
      // slice, the slice's fragments read right after it.
#pragma unroll
      for (int s = 0; s < STAGES - 1; ++s) issue(s);
      for (int kt = 0; kt < nk; ++kt) {
        // Slice kt has landed (this wave's DMA; the barrier covers the other
        // waves'), and every wave has consumed its reads of slice kt-1, whose
        // buffer the next issue refills.  lds_barrier, not __syncthreads:
        // the later slices' DMA stays in flight.
        wait_vmcnt<LOADS_PER_SLICE * (STAGES - 2)>();
        lds_barrier();
        issue(kt + STAGES - 1);
        const char *st = lds + (kt % STAGES) * STAGE_BYTES;
        u32x4 fa[2][MI], fb[2][NJ];
        read_frags(st, 0, fa[0], fb[0]);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          if constexpr (ASM_READS) wait_lgkm0_fenced();  // k-step ks's fragments, nothing newer yet
          if (ks + 1 < KSTEPS) read_frags(st, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
          mfmas(fa[ks & 1], fb[ks & 1]);
        }
      }
    }

    wait_vmcnt<0>();  // the trailing (all out-of-range) DMA has landed before the LDS is released
    // The last slice's schedule may leave fragment reads of a slice that does
    // not exist in flight; their registers are dead, and the epilogue may
    // reuse them for addresses, so those reads must land first.
    wait_lgkm0_fenced();
  }
};

// Producer/consumer tile: the warp-specialised design of "Warp
// Specialization HGEMM: 生产者-消费者模型的 GPU 形态" (section 问题的本质 and
// the summary: copy warps only move tiles into a shared-memory ring, compute
// warps only run the matrix instructions, and the two sides hand ring slots
// to each other), built for gfx950:
//   * four producer waves only issue the LDS DMA (buffer_load ... lds) of
//     every slice into a STAGES-deep ring and wait for it to land; four
//     consumer waves only read fragments (ds_read) and issue MFMAs.  A
//     producer whose DMA cannot issue yet (the CU's load path is full) stalls
//     alone: the consumer on its SIMD keeps the matrix pipe busy, whereas a
//     wave that does both stalls its own MFMAs behind the blocked load;
//   * the hand-off is gfx950's workgroup barrier, once per slice (the pages'
//     per-slot full/empty barriers have no gfx950 counterpart; a single
//     barrier carries both directions): between barriers i and i + 1 the
//     consumers run slice i's MFMAs from registers and read slice i + 1's
//     fragments, while the producers refill slot i % STAGES (slice i was read
//     before barrier i; slice 0, read after barrier 0, has a barrier of its
//     own) with slice i + STAGES and wait until slice i + 2 has landed, so
//     STAGES - 2 slices of DMA stay in flight at every barrier;
//   * every wave of a kernel gets the same register allocation, so the tile
//     is sized for consumers of at most 256 registers: 256 x 128 or
//     128 x 256 with 2 x 2 consumer waves of 128 x 64 or 64 x 128 (128
//     accumulators per lane), eight waves in all, one producer and one
//     consumer per SIMD.
// Tails and slices past the last one are handled as in DmaTile (out-of-range
// offsets write zeros).
template <typename TI, typename TO, int BM_, int BN_, int BK_, int STAGES_, int CWM, int CWN, bool A_KC,
          bool B_KC>
struct WsTile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_;
  static constexpr int NC = CWM * CWN, NP = 4, NW = NC + NP, NT = 64 * NW;
  static constexpr int ES = sizeof(TI);
  using OA = DmaOperand<BM, BK, A_KC, NP, ES>;
  using OB = DmaOperand<BN, BK, B_KC, NP, ES>;
  static constexpr int A_BYTES = OA::BYTES, B_BYTES = OB::BYTES;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int A_INST = OA::INST, B_INST = OB::INST;
  static constexpr int LOADS = A_INST + B_INST;  // DMA instructions per producer wave per slice
  static constexpr int WTM = BM / CWM, WTN = BN / CWN;
  static constexpr int MI = WTM / 16, NJ = WTN / 16;
  static constexpr int RD_B = NJ * OB::READS, RD_A = MI * OA::READS, RD = RD_A + RD_B;
  static constexpr int MFMAS = MI * NJ;
  static constexpr int PO = (RD + MFMAS - 1) / MFMAS;  // fragment reads after each MFMA
  static_assert(ES == 2 && BK * ES == 64, "16-bit inputs, one k-step (32 k) per slice");
  static_assert(NC == 4, "four consumer waves, one per SIMD next to one producer");
  static_assert(STAGES >= 3 && STAGES * STAGE_BYTES <= 160 * 1024, "ring depth and LDS budget");
  static_assert(LOADS * (STAGES - 2) < 64, "vmcnt range");

  static __device__ __forceinline__ void run(const GemmParams &p) {
    __shared__ __attribute__((aligned(1024))) char lds[STAGES * STAGE_BYTES];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tm, tn, kb, K;
    work_coords(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, p.splits, p.K, p.k_chunk, tm, tn, kb, K);
    const int m0 = tm * BM, n0 = tn * BN;
    const int nk = (K + BK - 1) / BK;  // >= 1: K == 0 never reaches a tile kernel

    if (wave >= NC) {  // ---------------------------------------- producer
      const int pw = wave - NC;
      const char *Ab = static_cast<const char *>(p.A) +
                       (A_KC ? (int64_t)m0 * p.lda + kb : (int64_t)kb * p.lda + m0) * ES;
      const char *Bb = static_cast<const char *>(p.B) +
                       (B_KC ? (int64_t)n0 * p.ldb + kb : (int64_t)kb * p.ldb + n0) * ES;
      const int64_t a_step = (A_KC ? BK : (int64_t)BK * p.lda) * ES;
      const int64_t b_step = (B_KC ? BK : (int64_t)BK * p.ldb) * ES;
      const uint32_t lda_b = (uint32_t)(p.lda * ES), ldb_b = (uint32_t)(p.ldb * ES);
      const int rva = p.M - m0, rvb = p.N - n0;
      auto issue = [&](int kt) {  // slice kt into slot kt % STAGES; past the last slice: zeros, no reads
        char *st = lds + (kt % STAGES) * STAGE_BYTES;
        const int kv = K - kt * BK;
#pragma unroll
        for (int u = 0; u < A_INST; ++u) OA::dma(make_rsrc(Ab + kt * a_step), lda_b, rva, kv, st, pw, lane, u);
#pragma unroll
        for (int u = 0; u < B_INST; ++u)
          OB::dma(make_rsrc(Bb + kt * b_step), ldb_b, rvb, kv, st + A_BYTES, pw, lane, u);
      };
#pragma unroll
      for (int s = 0; s < STAGES; ++s) issue(s);
      wait_vmcnt<LOADS * (STAGES - 2)>();  // slices 0 and 1 have landed
      lds_barrier();                       // barrier 0
      lds_barrier();                       // the consumers hold slice 0's fragments: slot 0 may be refilled
      for (int i = 0; i < nk; ++i) {
        issue(i + STAGES);                   // slot i % STAGES: slice i was read before barrier i
        wait_vmcnt<LOADS * (STAGES - 2)>();  // slice i + 2 has landed
        lds_barrier();                       // barrier i + 1
      }
      wait_vmcnt<0>();  // the trailing (all out-of-range) DMA has landed before the LDS is released
      return;
    }

    // ----------------------------------------------------------- consumer
    const int wm = wave / CWN, wn = wave % CWN;
    f32x4 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    typename OA::template Frag<MI, 1> fra;
    typename OB::template Frag<NJ, 1> frb;
    fra.init(lane, wm * MI);
    frb.init(lane, wn * NJ);
    auto read_op = [&](const char *st, int t, u32x4 (&fa)[MI], u32x4 (&fb)[NJ]) {
      if (t < RD_B) frb.read(st + A_BYTES, t / OB::READS, 0, t % OB::READS, fb[t / OB::READS]);
      else fra.read(st, (t - RD_B) / OA::READS, 0, (t - RD_B) % OA::READS, fa[(t - RD_B) / OA::READS]);
    };
    u32x4 fa[2][MI], fb[2][NJ];
    lds_barrier();  // barrier 0: slices 0 and 1 are in LDS
#pragma unroll
    for (int t = 0; t < RD; ++t) read_op(lds, t, fa[0], fb[0]);
    wait_lgkm0_fenced();
    lds_barrier();  // slice 0's fragments are in registers: the producers may refill slot 0
    for (int i = 0; i < nk; i += 2) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {  // two slices per trip keep the fragment buffers static
        const int k = i + h;
        const char *nx = lds + ((k + 1) % STAGES) * STAGE_BYTES;
        const bool more = k + 1 < nk;
#pragma unroll
        for (int t = 0; t < MFMAS; ++t) {
          const int ii = t / NJ, jj = t % NJ;
          Mfma<TI>::step(acc[ii][jj], fb[h][jj], fa[h][ii]);
#pragma unroll
          for (int o = t * PO; o < (t + 1) * PO; ++o)
            if (o < RD && more) read_op(nx, o, fa[h ^ 1], fb[h ^ 1]);
          __builtin_amdgcn_sched_barrier(0);
        }
        wait_lgkm0_fenced();  // slice k + 1's fragments are in registers; slot k % STAGES is no longer read
        lds_barrier();        // barrier k + 1
        if (!more) break;
      }
    }
    if (p.splits > 1)
      GemmEpilogue<float, MI, NJ>::store(partial_params(p, kb), acc, m0 + wm * WTM, n0 + wn * WTN, lane);
    else
      GemmEpilogue<TO, MI, NJ>::store(p, acc, m0 + wm * WTM, n0 + wn * WTN, lane);
  }
};

template <class Tile>
__global__ void __launch_bounds__(Tile::NT) gemm_dma_kernel(GemmParams p) {
  Tile::run(p);
}

}  // namespace mg
