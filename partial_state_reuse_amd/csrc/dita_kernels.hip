// HIP kernels of the dita library for gfx950 (CDNA4, wave64).
//
// One step of partitioned attention with selective attention-state reuse (DiTango,
// gist.science 2607.15650, "State-Centric Parallel Runtime / Composizione dello Stato"):
// for query partition i, every non-skipped key partition j contributes a state
// (O_ij, lse_ij); fresh states are recomputed from this step's Q/K/V and written to their
// cache slot, reused states are read from the slot, and all states of a row are merged by
// log-sum-exp (associative and commutative, so the order is free).
//
// Kernels
//   transpose_v     V [B,H,N,D] bf16 -> V^T scratch [B*H][DP][kt_pad] fp16, each partition's
//                   key range padded with zeros to a multiple of the key tile.
//   step_bf16<DP, MEASURE, FP8, FIXED>
//                   one workgroup (4 waves) per (b, h, query partition i, row tile), per
//                   pack of tail sub-tiles, or per part of a split row tile (the plan's list
//                   of workgroups).  For each fresh j: flash-attention over j's keys with MFMA
//                   (S^T = K Q^T in bf16, then O^T += V^T P^T in fp16), K and V^T tiles
//                   staged through LDS; at the block's end the normalised state goes to the
//                   cache (bf16 or fp8 O, f32 lse) and is folded into the row's running
//                   merge.  For each reused j the cached state is streamed with 16-byte loads
//                   and folded the same way.  The epilogue writes out = acc / l (f32) and the
//                   row lse.  MEASURE adds the planner's measurement of the diagonal states'
//                   change, for steps that take no snapshot of them (otherwise diag_change
//                   measures after the step); FIXED is the fixed-reference pass (below),
//                   after which the FIXED = false kernel runs as a conditional second pass.
//   merge_splits    after each pass: the parts' partial merges of each split row tile
//                   combined, and its rows written.
//   step_f32        the same computation in plain fp32 VALU arithmetic, one lane per row.
//   snapshot_diag   the diagonal slots copied aside before a measuring bf16 step.
//   diag_change     after it, the diagonal states' squared change against that copy.
//   planner_delta, planner_weights_part, planner_weights_sum
//                   the planner's growth (per partition) and importance (per block) sums.
//   merge_slots     group composition: cached states of a key group merged into one slot.
//   read_slot       copies one cache slot out in plain row-major layout.
//
// Register layout of the bf16 kernel.  The 32x32x16 bf16 MFMA produces a 32x32 f32 tile in
// which lane l holds column l%32 and rows 8*(r/4) + 4*(l/32) + r%4 for its 16 registers r.
// With S^T = K Q^T every lane therefore holds 16 keys of ONE query (l%32), so row max and
// row sum are in-lane plus one exchange between lanes l and l^32, and O^T = V^T P^T keeps
// the same one-query-per-lane layout, so the softmax rescale factors never cross lanes.
// K rows are fed to the MFMA in the order pi(rho) (bits 2 and 3 of the row index swapped),
// which makes the 8 keys each lane contributes to the P^T operand contiguous, so the V^T
// operand is one 16-byte LDS read.
#include <hip/hip_runtime.h>

#include <mutex>
#include <stdint.h>

#include "dita_internal.h"

namespace dita {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// element offset of head (b, h) = (bh / H, bh % H) in Q, K, V and out
__device__ __forceinline__ size_t head_base(const StepArgs& a, int bh) {
  const int b = bh / a.H, h = bh - b * a.H;
  return (size_t)b * a.sB + (size_t)h * a.sH;
}
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// max / sum of the values held by lanes l and l^32, in every lane, through ds_bpermute with
// the partner's byte address precomputed once.  (v_permlane32_swap would avoid the LDS
// crossbar, but the compiler substitutes one of its two results for the other when both
// operands hold the same value, which silently drops the exchange.)
__device__ __forceinline__ int partner_addr() { return (int)((__lane_id() ^ 32u) << 2); }
__device__ __forceinline__ float from_partner(float x, int addr) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(addr, __builtin_bit_cast(int, x)));
}
__device__ __forceinline__ float max_halves(float x, int addr) {
  return fmaxf(x, from_partner(x, addr));
}
__device__ __forceinline__ float sum_halves(float x, int addr) {
  return x + from_partner(x, addr);
}

// The device plan is written by the host before the launch and never by a kernel, so it is
// read through the constant address space: uniform reads become scalar loads, which are
// counted separately from the vector loads in flight (a vector read of the plan would make
// the wave wait for every outstanding prefetch).
typedef __attribute__((address_space(4))) const int32_t cint;
__device__ __forceinline__ const cint* as_const(const int32_t* p) { return (const cint*)p; }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }
// A raw buffer resource over the bytes [base, base + bytes) (bytes above 2^32 - 1 clamped):
// a load through it takes a wave-uniform base and a 32-bit per-lane byte offset (no 64-bit
// address arithmetic), and a load at an offset past the end returns zeros.  Word 3 is the
// raw-buffer setting of the gfx9 family.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = (uint32_t)(bytes >> 32) != 0u ? 0xffffffffu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)n, 0x00020000);
}
__device__ __forceinline__ u32x4 buf16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *(u32x4*)p = v; }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

// S^T row index rho -> key position inside a 32-key half: swap bits 2 and 3.
__device__ __forceinline__ int key_of_row(int rho) {
  return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1);
}

// XCD-aware workgroup order: consecutive workgroup ids are dealt round-robin to the 8 XCDs;
// remap so that each XCD walks a contiguous range of logical work (same head, adjacent rows),
// which keeps the K/V partitions it shares in that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int G) {
  const int xcd = bid & 7, idx = bid >> 3, per = G >> 3, rem = G & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

// ------------------------------------------------------------------------------------------
// zero the device counters
// ------------------------------------------------------------------------------------------
__global__ void zero_u64(unsigned long long* p, int n) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n) p[t] = 0ull;
}

// ------------------------------------------------------------------------------------------
// V [B,H,N,D] bf16 -> V^T [B*H][DP][kt_pad] fp16, zero padded.  Every bf16 value of fp16 range
// converts exactly (8 significant bits fit in 11; magnitudes below 2^-14 keep an absolute
// error under 2^-25).  Values beyond the fp16 range are counted in counters[2].
// grid (kt_pad / 64, B*H), block 256
// ------------------------------------------------------------------------------------------
constexpr float kF16Max = 65504.0f;

__global__ __launch_bounds__(256) void transpose_v(StepArgs a) {
  __shared__ uint16_t tile[64][129];   // 64 keys x up to 128 dims of fp16 (+1 against conflicts)
  const int bh = blockIdx.y;
  const int col0 = blockIdx.x * 64;    // padded key index
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) a.counters[4] = 0;
  const int* poffs = a.plan + a.off_poffs;
  const int* offs = a.plan + a.off_offs;
  // partition of this 64-key chunk (poffs are multiples of 64)
  int lo = 0, hi = a.P - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (poffs[mid] <= col0) lo = mid; else hi = mid - 1;
  }
  const int p = lo;
  const int o_p = offs[p], n_p = offs[p + 1] - o_p;
  const int k0 = col0 - poffs[p];      // first key (partition-relative)
  const uint16_t* V = (const uint16_t*)a.v + head_base(a, bh);
  // load 64 keys x D (8 elements per 16-byte chunk), converting to fp16
  const int cpr = a.D / 8;             // chunks per row
  int out_of_range = 0;
  for (int c = threadIdx.x; c < 64 * cpr; c += 256) {
    const int r = c / cpr, d8 = (c - r * cpr) * 8;
    const int key = k0 + r;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (key < n_p) val = ld16(V + (size_t)(o_p + key) * a.ld + d8);
    const bf16x8 b = as_bf16x8(val);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float f = (float)b[t];
      out_of_range += !(fabsf(f) <= kF16Max);
      tile[r][d8 + t] = __builtin_bit_cast(uint16_t, (_Float16)f);
    }
  }
  if (out_of_range) atomicAdd(&a.counters[2], (unsigned long long)out_of_range);
  __syncthreads();
  // write DP rows x 64 keys, 8 keys per 16-byte chunk
  uint16_t* VT = (uint16_t*)a.vt + (size_t)bh * a.DP * a.kt_pad;
  for (int c = threadIdx.x; c < a.DP * 8; c += 256) {
    const int d = c >> 3, c8 = (c & 7) * 8;
    u32x4 val;
    uint16_t* e = (uint16_t*)&val;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int key = k0 + c8 + t;
      e[t] = (d < a.D && key < n_p) ? tile[c8 + t][d] : (uint16_t)0;
    }
    st16(VT + (size_t)d * a.kt_pad + col0 + c8, val);
  }
}

// ------------------------------------------------------------------------------------------
// bf16 fused step.  Each wave works on a 32-row sub-tile of one query partition (lane l:
// query row l%32).  Two kinds of workgroup, 4 waves each:
//   group: the 4 waves take 128 consecutive rows of one partition and share every K / V^T
//          tile, staged in LDS;
//   tail:  one sub-tile left over at the end of a partition; the 4 waves split its blocks,
//          read their K / V^T fragments straight from global memory, and combine their
//          partial merges through LDS at the end.
// ------------------------------------------------------------------------------------------
// Lazy rescale: the running reference m of a block state is raised only when a new logit
// exceeds it by more than this many powers of two, so p = 2^(s - m) stays <= 2^8 and the
// accumulator is rescaled rarely (the result is exact either way: m is only a reference).
constexpr float kRescaleSlack = 8.0f;
// Fixed reference (FIXED instantiation, launched when every fresh block's slot holds its state
// from an earlier step): each row takes that state's lse (base 2) minus kRefHeadroom as its
// reference for the whole block, with no running maximum; consecutive steps' inputs differ
// little, so the row sum lands near 2^kRefHeadroom.  A row sum outside [kRefLo, kRefHi] (some
// p above 2^15, which fp16 cannot be trusted to hold, or the block's mass more than 6 powers
// of two below the reference, where fp16 loses its small p) rejects the pass: it raises the
// step's flag, and the running-maximum kernel, launched after it as a conditional second
// pass, computes the whole step again.
constexpr float kRefHeadroom = 8.0f;
constexpr float kRefLo = 4.0f;
constexpr float kRefHi = 32768.0f;

// Wave-wide sum (every lane gets the total), in a fixed butterfly order.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// fp8 e4m3 cache elements: 16 f32 values of a lane's fragment <-> 16 bytes, value r in byte
// r, with the hardware conversion (round to nearest even, saturating at +-448).
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x4 fp8_pack16(const f32x16& v) {
  u32x4 o;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * k], v[4 * k + 1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * k + 2], v[4 * k + 3], w, true);
    o[k] = (uint32_t)w;
  }
  return o;
}
__device__ __forceinline__ void fp8_unpack16(u32x4 w, float* v) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], true);
    v[4 * k] = lo[0];
    v[4 * k + 1] = lo[1];
    v[4 * k + 2] = hi[0];
    v[4 * k + 3] = hi[1];
  }
}
// element type of the cached O: bf16 bits, or fp8 bytes
template <bool FP8> struct CacheElem { typedef uint16_t type; };
template <> struct CacheElem<true> { typedef uint8_t type; };

// Block end, for the wave's 32-row sub-tile: normalise the block state, store it to its
// slot (O^T fragment as bf16 or fp8 in fragment order, lse as f32 natural log) and fold it into
// the row's running merge (base-2 units).  For a diagonal block with the planner measurement
// on, the squared change of the cached O (new - old, over rows < n_i and dims < D) is summed
// first and stored for the sub-tile.
template <int NDT, bool MEASURE, bool FP8>
__device__ __forceinline__ void block_end(const StepArgs& a, f32x16 (&bacc)[NDT], float m_b,
                                          float l_b, int paddr, size_t slot_base, int row0,
                                          int myrow, typename CacheElem<FP8>::type* dst,
                                          f32x16 (&acc)[NDT],
                                          float& m_row, float& l_row, bool diag, int n_i,
                                          int i, int bh) {
  typedef typename CacheElem<FP8>::type CT;
  const int lane = threadIdx.x & 63, h32 = lane >> 5;
  const float lsum = sum_halves(l_b, paddr);
  const float inv = 1.0f / lsum;
  const float lse2 = m_b + fast_log2(lsum);      // block lse, base 2
  const bool measure = MEASURE && diag;                    // wave-uniform
  // the old state: the step's snapshot of the diagonal slots, else the slot itself
  const CT* old = MEASURE && a.diag_snap
      ? (const CT*)a.diag_snap + ((size_t)bh * a.P + i) * ((size_t)a.slot_rows * NDT * 32) +
            (size_t)row0 * NDT * 32
      : dst;
  float sq = 0.f;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    bacc[dt] *= inv;
    if constexpr (FP8) {
      const u32x4 w = fp8_pack16(bacc[dt]);
      if (measure) {
        float nv[16], ov[16];
        fp8_unpack16(w, nv);
        fp8_unpack16(ld16(old + dt * 1024 + lane * 16), ov);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int d = dt * 32 + 8 * (r >> 2) + 4 * h32 + (r & 3);
          const float df = nv[r] - ov[r];
          if (myrow < n_i && d < a.D) sq = __builtin_fmaf(df, df, sq);
        }
      }
      st16(dst + dt * 1024 + lane * 16, w);
      continue;
    }
    u32x4 w0, w1;
    uint16_t* e0p = (uint16_t*)&w0;
    uint16_t* e1p = (uint16_t*)&w1;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      e0p[r] = __builtin_bit_cast(uint16_t, (__bf16)bacc[dt][r]);
      e1p[r] = __builtin_bit_cast(uint16_t, (__bf16)bacc[dt][r + 8]);
    }
    if (measure) {
      const u32x4 o0 = ld16(old + dt * 1024 + lane * 16), o1 = ld16(old + dt * 1024 + lane * 16 + 8);
      const bf16x8 n0 = as_bf16x8(w0), n1 = as_bf16x8(w1), p0 = as_bf16x8(o0), p1 = as_bf16x8(o1);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // accumulator row r of d tile dt holds d = dt*32 + 8*(r/4) + 4*h32 + r%4
        const int d = dt * 32 + 8 * (r >> 2) + 4 * h32 + (r & 3);
        const float df = r < 8 ? (float)n0[r] - (float)p0[r] : (float)n1[r - 8] - (float)p1[r - 8];
        if (myrow < n_i && d < a.D) sq = __builtin_fmaf(df, df, sq);
      }
    }
    st16(dst + dt * 1024 + lane * 16, w0);
    st16(dst + dt * 1024 + lane * 16 + 8, w1);
  }
  if (measure) {
    sq = wave_sum(sq);
    if (lane == 0) a.delta_part[((size_t)bh * a.P + i) * a.delta_stride + (row0 >> 5)] = sq;
  }
  if (h32 == 0) a.cache_lse[slot_base * a.slot_rows + myrow] = lse2 * kLn2;
  const float mn = fmaxf(m_row, lse2);
  const float fa = fast_exp2(m_row - mn), fb = fast_exp2(lse2 - mn);
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = acc[dt] * fa + bacc[dt] * fb;
  l_row = l_row * fa + fb;
  m_row = mn;
}

// Reused states e_begin, e_begin + STEP, ... (below e_end) folded into the row's merge, for
// the wave's 32-row sub-tile.
template <int DP, bool FP8, int STEP>
__device__ __forceinline__ void reuse_fold(const StepArgs& a, int bh, int row0, int e0,
                                           int e_begin, int e_end, f32x16 (&acc)[DP / 32],
                                           float& m_row, float& l_row) {
  constexpr int NDT = DP / 32;
  const int lane = threadIdx.x & 63, l32 = lane & 31;
  const int myrow = row0 + l32;
  const cint* ent = as_const(a.plan) + a.off_ent;
  const size_t slot_elems = (size_t)a.slot_rows * DP;
  typedef typename CacheElem<FP8>::type CT;
  const CT* cache_o = (const CT*)a.cache_o;
  // The reused states are taken RB at a time: their loads are all issued before the first
  // of them is folded, so a wave waits for one memory round trip per RB states.
  constexpr int RB = 4;
  constexpr int NW = FP8 ? 1 : 2;               // 16-byte words per lane per d tile
  for (int e = e_begin; e < e_end; e += RB * STEP) {
    u32x4 raw[RB][NDT][NW];
    float lse2[RB];
#pragma unroll
    for (int q = 0; q < RB; ++q) {
      if (e + q * STEP < e_end) {                 // wave-uniform
        const int slot = ent[2 * (e0 + e + q * STEP) + 1];
        const size_t slot_base = (size_t)bh * a.num_slots + slot;
        lse2[q] = a.cache_lse[slot_base * a.slot_rows + myrow];
        const CT* src = cache_o + slot_base * slot_elems + (size_t)row0 * DP;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int w = 0; w < NW; ++w) raw[q][dt][w] = ld16(src + dt * 1024 + lane * 16 + w * 8);
      }
    }
#pragma unroll
    for (int q = 0; q < RB; ++q) {
      if (e + q * STEP < e_end) {
        const float l2 = lse2[q] * kLog2e;
        const float mn = fmaxf(m_row, l2);
        const float fa = fast_exp2(m_row - mn), fb = fast_exp2(l2 - mn);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          float v[16];
          if constexpr (FP8) {
            fp8_unpack16(raw[q][dt][0], v);
          } else {
            const bf16x8 lo = as_bf16x8(raw[q][dt][0]), hi = as_bf16x8(raw[q][dt][NW - 1]);
#pragma unroll
            for (int r = 0; r < 8; ++r) {
              v[r] = (float)lo[r];
              v[r + 8] = (float)hi[r];
            }
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[dt][r] = acc[dt][r] * fa + v[r] * fb;
        }
        l_row = l_row * fa + fb;
        m_row = mn;
      }
    }
  }
}

// The epilogue (out = acc / l, lse) and the per-partition block counts, for the wave's
// 32-row sub-tile.
template <int DP>
__device__ __forceinline__ void finish_rows(const StepArgs& a, int bh, int o_i, int n_i,
                                            int row0, int nf, int nr,
                                            const f32x16 (&acc)[DP / 32], float m_row,
                                            float l_row) {
  constexpr int NDT = DP / 32;
  const int lane = threadIdx.x & 63, h32 = lane >> 5, l32 = lane & 31;
  const int myrow = row0 + l32;
  const size_t bhN = (size_t)bh * a.N;
  if (myrow < n_i) {
    const float inv = 1.0f / l_row;
    const size_t orow = head_base(a, bh) + (size_t)(o_i + myrow) * a.ld;   // element offset
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = dt * 32 + 8 * q4 + 4 * h32;
        if (d < a.D) {
          f32x4 v = {acc[dt][4 * q4] * inv, acc[dt][4 * q4 + 1] * inv,
                     acc[dt][4 * q4 + 2] * inv, acc[dt][4 * q4 + 3] * inv};
          if (a.out_bf16) {                       // uniform: 4 values rounded to bf16, 8 bytes
            uint16_t e[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) e[t] = __builtin_bit_cast(uint16_t, (__bf16)v[t]);
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            const u32x2 w = {(uint32_t)e[0] | ((uint32_t)e[1] << 16),
                             (uint32_t)e[2] | ((uint32_t)e[3] << 16)};
            *(u32x2*)((uint16_t*)a.out + orow + d) = w;
          } else {
            *(f32x4*)((float*)a.out + orow + d) = v;
          }
        }
      }
    }
    if (a.lse_out && h32 == 0)
      a.lse_out[bhN + o_i + myrow] = (m_row + fast_log2(l_row)) * kLn2;
  }
  // block counts, once per partition row: by the wave that holds its first rows
  if (row0 == 0 && lane == 0 && !a.fixup) {
    atomicAdd(&a.counters[0], (unsigned long long)nf);
    atomicAdd(&a.counters[1], (unsigned long long)nr);
  }
}

// Tail workgroup k: a pack of tail sub-tiles -- the rows left at the ends of consecutive
// partitions, at most 32 in all -- whose lane l holds row r_l of partition i_l (its member's
// rows follow one another over the lanes; lanes past the pack's rows hold none).  The 4
// waves go through the union of the members' fresh blocks together, splitting each block's
// keys (wave w takes every 4th 32-key unit from the w-th), over all 32 rows; the four
// partial states of a block are merged exactly (any order) through LDS by wave 0, and a lane
// keeps the block only where it is fresh for its own partition, storing the state to that
// block's slot and folding it into its row's merge.  Reused states are split over the waves
// (entry e of each row's reuse list for e = w, w + 4, ...), every lane reading its own
// partition's slot.  K / V^T fragments come straight from global memory (L2); the partial
// merges are combined through LDS (exact in any order) and wave 0 writes the rows.  `lds`
// holds 4 slots of 64 x (2 + DP / 2) floats.
template <int DP, bool MEASURE, bool FP8>
__device__ __forceinline__ void tail_pack(const StepArgs& a, int bh, int k, float* lds) {
  constexpr int NKC = DP / 16, NDT = DP / 32;
  typedef typename CacheElem<FP8>::type CT;
  // the wave index as a scalar, so that LDS addresses split into a scalar base and a per-lane
  // offset with the element index as an immediate
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h32 = lane >> 5, l32 = lane & 31;
  const cint* plan = as_const(a.plan);
  const cint* offs = plan + a.off_offs;
  const cint* poffs = plan + a.off_poffs;
  const cint* pk = plan + a.off_pack + 4 * k;
  const int m0 = pk[0], nm = pk[1], u0 = pk[2], nu = pk[3];
  // this lane's member (pack index), partition and row
  int mem = 0, i = 0, r = 0, rfirst = 0;
  bool valid = false;
  for (int m = 0; m < nm; ++m) {                 // uniform loop, per-lane choice
    const cint* me = plan + a.off_member + 4 * (m0 + m);
    const int lane0 = me[3], rows = me[2];
    if (l32 >= lane0 && l32 < lane0 + rows) {
      mem = m;
      i = me[0];
      r = me[1] + (l32 - lane0);
      rfirst = me[1];
      valid = true;
    }
  }
  const int* offs_v = a.plan + a.off_offs;        // per-lane reads of the plan
  const int* rinfo = a.plan + a.off_rows + 4 * i;
  const int o_i = offs_v[i];
  const int e0 = rinfo[0], nf = rinfo[1], nr = valid ? rinfo[2] : 0;
  const cint* uent = plan + a.off_union;
  const int* pslot = a.plan + a.off_pslot;
  const int* ent_v = a.plan + a.off_ent;
  const float sc = a.scale_log2;
  const float inv_sc = 1.0f / sc;
  const int paddr = partner_addr();
  const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  // this lane's position in a slot's fragment order: sub-tile r / 32, lane (h32, r % 32)
  const size_t frag = (size_t)(r & ~31) * DP + (size_t)(h32 * 32 + (r & 31)) * 16;

  bf16x8 qf[NKC];
  {
    const uint16_t* Q = (const uint16_t*)a.q + head_base(a, bh);
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const int d0 = kc * 16 + h32 * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (valid && d0 < a.D) v = ld16(Q + (size_t)(o_i + r) * a.ld + d0);
      qf[kc] = as_bf16x8(v);
    }
  }
  // the row's merge: m, l in registers; during the fresh blocks wave 0 keeps O in LDS (in the
  // slot of partial states that it does not use, 16 NDT floats per lane), which leaves the
  // block loop the registers of its one-unit-ahead fragment loads
  float m_row = kNegInf, l_row = 0.f;
  float* racc = lds + lane;                      // slot 0 (wave 0 leaves no partial state)
  if (wave == 0) {
#pragma unroll
    for (int x = 0; x < NDT * 16; ++x) racc[x * 64] = 0.f;
  }
  const size_t slot_elems = (size_t)a.slot_rows * DP;
  CT* cache_o = (CT*)a.cache_o;
  const uint16_t* Kg = (const uint16_t*)a.k + head_base(a, bh);
  const uint16_t* VTg = (const uint16_t*)a.vt + (size_t)bh * DP * a.kt_pad;

  // ---------------- fresh blocks: the union of the members', one at a time ----------------
  // Wave w takes the 32-key units w, w + 4, ... of the block, each unit's K and V^T fragments
  // loaded one unit ahead (K after this unit's QK MFMAs, V^T after its PV MFMAs).  At the
  // block's end waves 1-3 leave their partial states in LDS and wave 0 merges them into its
  // own, then writes the block's state and folds it into the row's merge; waves 1-3 go on
  // with the next block meanwhile.
  constexpr int W = 2 + NDT * 16;               // floats per lane of a partial state
  for (int t = 0; t < nu; ++t) {
    const int j = uent[2 * (u0 + t)], sb = uent[2 * (u0 + t) + 1];
    const int o_j = offs[j], n_j = offs[j + 1] - o_j, po_j = poffs[j];
    const int nunits = (n_j + 31) >> 5;
    f32x16 bacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) bacc[dt] = (f32x16){};
    float m_b = kNegInf, l_b = 0.f, thr = kNegInf;
    bf16x8 kf[NKC];
    f16x8 vf[NDT][2];
    auto load_k = [&](int u) {
      const int key = min(u * 32 + key_of_row(l32), n_j - 1);
      const uint16_t* src = Kg + (size_t)(o_j + key) * a.ld;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) kf[kc] = as_bf16x8(ld16(src + min(kc * 16 + h32 * 8, a.D - 8)));
    };
    auto load_v = [&](int u) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          vf[dt][c] = as_f16x8(ld16(VTg + (size_t)(dt * 32 + l32) * a.kt_pad + po_j + u * 32 + c * 16 + h32 * 8));
    };
    if (wave < nunits) {
      load_k(wave);
      load_v(wave);
    }
    for (int u = wave; u < nunits; u += kWaves) {
      const int kbase = u * 32;
      f32x16 s = (f32x16){};
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kc], qf[kc], s, 0, 0, 0);
      const bool more = u + kWaves < nunits;    // wave-uniform
      if (more) load_k(u + kWaves);
      if (kbase + 32 > n_j) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int key = kbase + 16 * (q >> 3) + 8 * h32 + (q & 7);
          if (key >= n_j) s[q] = kNegInf;
        }
      }
      float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
      for (int q = 3; q < 16; q += 2) mx = fmaxf(fmaxf(mx, s[q]), s[q + 1 < 16 ? q + 1 : q]);
      // the rescale factor is applied on every unit (1 without a new maximum): a rescale
      // under a branch would keep two copies of the block accumulator live across it
      float alpha = 1.f;
      if (__any(mx > thr)) {
        const float m_new = fmaxf(m_b, max_halves(mx, paddr) * sc);
        alpha = fast_exp2(m_b - m_new);
        m_b = m_new;
        thr = (m_new + kRescaleSlack) * inv_sc;
      }
      l_b *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) bacc[dt] *= alpha;
      f16x8 pf[2];
#pragma unroll
      for (int q = 0; q < 16; ++q)
        pf[q >> 3][q & 7] = (_Float16)fast_exp2(__builtin_fmaf(s[q], sc, -m_b));
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          const f16x2 pair = {pf[c][2 * q2], pf[c][2 * q2 + 1]};
          l_b = __builtin_amdgcn_fdot2(pair, ones, l_b, false);
        }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          bacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[dt][c], pf[c], bacc[dt], 0, 0, 0);
      if (more) load_v(u + kWaves);
    }
    // the four partial states of the block, merged by wave 0 (a wave without keys holds
    // m = -inf, l = 0, O = 0, which the merge weights by 0)
    __syncthreads();                             // wave 0 has read the previous block's
    if (wave != 0) {
      float* p = lds + (size_t)wave * W * 64 + lane;
      p[0] = m_b;
      p[64] = l_b;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int x = 0; x < 16; ++x) p[(2 + dt * 16 + x) * 64] = bacc[dt][x];
    }
    __syncthreads();
    if (wave != 0) continue;
    {
      float mw[kWaves - 1];
      float mn = m_b;
#pragma unroll
      for (int w = 0; w < kWaves - 1; ++w) {
        mw[w] = lds[(size_t)(w + 1) * W * 64 + lane];
        mn = fmaxf(mn, mw[w]);
      }
      const float f0 = m_b == kNegInf ? 0.f : fast_exp2(m_b - mn);
      l_b *= f0;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) bacc[dt] *= f0;
#pragma unroll
      for (int w = 0; w < kWaves - 1; ++w) {
        const float* p = lds + (size_t)(w + 1) * W * 64 + lane;
        const float fw = mw[w] == kNegInf ? 0.f : fast_exp2(mw[w] - mn);
        l_b = __builtin_fmaf(p[64], fw, l_b);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int x = 0; x < 16; ++x) bacc[dt][x] = __builtin_fmaf(p[(2 + dt * 16 + x) * 64], fw, bacc[dt][x]);
      }
      m_b = mn;
    }
    const int slot = valid ? pslot[sb + mem] : -1;
    const bool mine = slot >= 0;                 // j is fresh for this lane's partition
    // block end, for the lanes whose partition has j fresh: the normalised state to the slot
    // (fragment order, at this lane's row), the lse, and the fold into the row's merge
    const float lsum = sum_halves(l_b, paddr);
    const float inv = 1.0f / lsum;
    const float lse2 = m_b + fast_log2(lsum);
    const bool diag = MEASURE && mine && j == i;
    const size_t sbase = (size_t)bh * a.num_slots + (mine ? slot : 0);
    CT* dst = cache_o + sbase * slot_elems + frag;
    const CT* old = MEASURE && a.diag_snap
        ? (const CT*)a.diag_snap + ((size_t)bh * a.P + i) * slot_elems + frag
        : dst;
    float sq = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      bacc[dt] *= inv;
      if constexpr (FP8) {
        const u32x4 w = fp8_pack16(bacc[dt]);
        if (diag) {
          float nv[16], ov[16];
          fp8_unpack16(w, nv);
          fp8_unpack16(ld16(old + dt * 1024), ov);
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int d = dt * 32 + 8 * (q >> 2) + 4 * h32 + (q & 3);
            const float df = nv[q] - ov[q];
            if (d < a.D) sq = __builtin_fmaf(df, df, sq);
          }
        }
        if (mine) st16(dst + dt * 1024, w);
      } else {
        u32x4 w0, w1;
        uint16_t* e0p = (uint16_t*)&w0;
        uint16_t* e1p = (uint16_t*)&w1;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          e0p[q] = __builtin_bit_cast(uint16_t, (__bf16)bacc[dt][q]);
          e1p[q] = __builtin_bit_cast(uint16_t, (__bf16)bacc[dt][q + 8]);
        }
        if (diag) {
          const bf16x8 n0 = as_bf16x8(w0), n1 = as_bf16x8(w1);
          const bf16x8 p0 = as_bf16x8(ld16(old + dt * 1024)), p1 = as_bf16x8(ld16(old + dt * 1024 + 8));
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int d = dt * 32 + 8 * (q >> 2) + 4 * h32 + (q & 3);
            const float df = q < 8 ? (float)n0[q] - (float)p0[q] : (float)n1[q - 8] - (float)p1[q - 8];
            if (d < a.D) sq = __builtin_fmaf(df, df, sq);
          }
        }
        if (mine) {
          st16(dst + dt * 1024, w0);
          st16(dst + dt * 1024 + 8, w1);
        }
      }
    }
    if constexpr (MEASURE) {
      // the diagonal member's squared change: one sub-tile of partition j
      const unsigned long long dm = __ballot(diag);
      if (dm) {
        sq = wave_sum(sq);
        if (lane == (int)__builtin_ctzll(dm))
          a.delta_part[((size_t)bh * a.P + j) * a.delta_stride + (rfirst >> 5)] = sq;
      }
    }
    if (mine) {
      if (h32 == 0) a.cache_lse[sbase * a.slot_rows + r] = lse2 * kLn2;
      const float mn = fmaxf(m_row, lse2);
      const float fa = fast_exp2(m_row - mn), fb = fast_exp2(lse2 - mn);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int x = 0; x < 16; ++x)
          racc[(dt * 16 + x) * 64] = racc[(dt * 16 + x) * 64] * fa + bacc[dt][x] * fb;
      l_row = l_row * fa + fb;
      m_row = mn;
    }
  }

  __syncthreads();                               // wave 0 has read the last block's partials
  f32x16 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int x = 0; x < 16; ++x) acc[dt][x] = wave == 0 ? racc[(dt * 16 + x) * 64] : 0.f;

  // ---------------- reused states: entry e of each row's list, e = wave, wave + 4, ... ----
  {
    int nr_max = nr;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) nr_max = max(nr_max, __shfl_xor(nr_max, off));
    constexpr int RB = 4;
    constexpr int NW = FP8 ? 1 : 2;
    for (int e = wave; e < nr_max; e += RB * kWaves) {
      u32x4 raw[RB][NDT][NW];
      float lse2[RB];
#pragma unroll
      for (int q = 0; q < RB; ++q) {
        const int ee = e + q * kWaves;
        if (ee < nr) {
          const int rslot = ent_v[2 * (e0 + nf + ee) + 1];
          const size_t rb = (size_t)bh * a.num_slots + rslot;
          lse2[q] = a.cache_lse[rb * a.slot_rows + r];
          const CT* src = cache_o + rb * slot_elems + frag;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int w = 0; w < NW; ++w) raw[q][dt][w] = ld16(src + dt * 1024 + w * 8);
        }
      }
#pragma unroll
      for (int q = 0; q < RB; ++q) {
        const int ee = e + q * kWaves;
        if (ee < nr) {
          const float l2 = lse2[q] * kLog2e;
          const float mn = fmaxf(m_row, l2);
          const float fa = fast_exp2(m_row - mn), fb = fast_exp2(l2 - mn);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            float v[16];
            if constexpr (FP8) {
              fp8_unpack16(raw[q][dt][0], v);
            } else {
              const bf16x8 lo = as_bf16x8(raw[q][dt][0]), hi = as_bf16x8(raw[q][dt][NW - 1]);
#pragma unroll
              for (int x = 0; x < 8; ++x) {
                v[x] = (float)lo[x];
                v[x + 8] = (float)hi[x];
              }
            }
#pragma unroll
            for (int x = 0; x < 16; ++x) acc[dt][x] = acc[dt][x] * fa + v[x] * fb;
          }
          l_row = l_row * fa + fb;
          m_row = mn;
        }
      }
    }
  }

  // combine the partial merges: waves 2, 3 into 0, 1, then 1 into 0 (slot s of LDS holds the
  // merge of wave s)
  auto put = [&](int sl) {
    float* p = lds + (size_t)sl * W * 64 + lane;
    p[0] = m_row;
    p[64] = l_row;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int x = 0; x < 16; ++x) p[(2 + dt * 16 + x) * 64] = acc[dt][x];
  };
  auto take = [&](int sl) {
    const float* p = lds + (size_t)sl * W * 64 + lane;
    const float m2 = p[0], l2 = p[64];
    const float mn = fmaxf(m_row, m2);
    const float fa = m_row == kNegInf ? 0.f : fast_exp2(m_row - mn);
    const float fb = m2 == kNegInf ? 0.f : fast_exp2(m2 - mn);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int x = 0; x < 16; ++x) acc[dt][x] = acc[dt][x] * fa + p[(2 + dt * 16 + x) * 64] * fb;
    l_row = l_row * fa + l2 * fb;
    m_row = mn;
  };
  if (wave >= 2) put(wave);
  __syncthreads();
  if (wave < 2) take(wave + 2);
  __syncthreads();
  if (wave == 1) put(1);
  __syncthreads();
  if (wave != 0) return;
  take(1);
  if (valid) {
    const float inv = 1.0f / l_row;
    const size_t orow = head_base(a, bh) + (size_t)(o_i + r) * a.ld;   // element offset
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = dt * 32 + 8 * q4 + 4 * h32;
        if (d < a.D) {
          f32x4 v = {acc[dt][4 * q4] * inv, acc[dt][4 * q4 + 1] * inv,
                     acc[dt][4 * q4 + 2] * inv, acc[dt][4 * q4 + 3] * inv};
          if (a.out_bf16) {
            uint16_t e[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) e[t] = __builtin_bit_cast(uint16_t, (__bf16)v[t]);
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            const u32x2 w = {(uint32_t)e[0] | ((uint32_t)e[1] << 16),
                             (uint32_t)e[2] | ((uint32_t)e[3] << 16)};
            *(u32x2*)((uint16_t*)a.out + orow + d) = w;
          } else {
            *(f32x4*)((float*)a.out + orow + d) = v;
          }
        }
      }
    }
    if (a.lse_out && h32 == 0)
      a.lse_out[(size_t)bh * a.N + o_i + r] = (m_row + fast_log2(l_row)) * kLn2;
    // block counts, once per partition: by the lane holding its first row, if it is a tail row
    if (r == 0 && h32 == 0 && !a.fixup) {
      atomicAdd(&a.counters[0], (unsigned long long)nf);
      atomicAdd(&a.counters[1], (unsigned long long)nr);
    }
  }
}

// MEASURE: the planner's measurement of the diagonal states' change is compiled in (a
// separate instantiation, so that steps without it keep the leaner register allocation); used
// only where no snapshot of the old diagonal states is taken, since with one the step runs
// the plain kernel and diag_change measures afterwards.
// FP8: the cached O is fp8 e4m3 instead of bf16.
// FIXED: the fixed-reference pass (row groups only; tail workgroups keep the running maximum).
// Occupancy: 3 waves per SIMD at D <= 64 (168 VGPRs); 2 at D = 96 and 128, where the register
// cap of 256 costs a few spills at block end only, and the second wave hides the latency
// the single wave left exposed (the D = 128 step is about a quarter faster than at 1 wave).
template <int DP, bool MEASURE, bool FP8, bool FIXED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DP == 64 ? 3 : 2))) void step_bf16(StepArgs a) {
  constexpr int NKC = DP / 16;        // 16-wide d chunks of Q K^T
  constexpr int NDT = DP / 32;        // 32-row d tiles of O^T
  constexpr int KT = kKeyTile;        // keys per LDS tile
  constexpr int NKS = KT / 32;        // 32-key halves per tile
  constexpr int LDK = DP + 8;         // LDS row stride of the K tile (elements)
  constexpr int LDV = KT + 8;         // LDS row stride of the V^T tile (elements)
  constexpr int CHK = KT * DP / 8 / 256;   // 16-byte chunks per thread per K tile
  constexpr int CHV = DP * KT / 8 / 256;   // ... per V^T tile
  constexpr int WG_ROWS = kWaves * 32;
  constexpr bool AHEAD = DP == 64;    // LDS fragment reads issued ahead of their MFMAs
  // K tile, then V^T tile; the tail workgroups use the same memory for one slot of 2 + DP / 2
  // floats per lane and wave (partial states and merges).  At DP >= 96 (2 waves per SIMD,
  // 256 VGPRs) the row groups keep the d tiles dt >= AF of the row's running merge in LDS
  // after the tiles between block ends (16 floats per lane and d tile), which frees their
  // registers in the tile loop; at DP = 64 all of it stays in registers (AF = NDT).
  constexpr int TILE_ELEMS = KT * LDK + DP * LDV;
  constexpr int MERGE_ELEMS = kWaves * (2 + DP / 2) * 64 * 2;
  constexpr int AF = DP >= 96 ? 2 : NDT;
  constexpr int ACC_ELEMS = kWaves * 64 * (NDT - AF) * 16 * 2;
  constexpr int RG_ELEMS = TILE_ELEMS + ACC_ELEMS;
  __shared__ __attribute__((aligned(16))) uint16_t smem[RG_ELEMS > MERGE_ELEMS ? RG_ELEMS : MERGE_ELEMS];
  uint16_t* const sK = smem;
  uint16_t* const sV = smem + KT * LDK;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h32 = lane >> 5, l32 = lane & 31;
  if (!FIXED && a.fixup) {                      // the conditional second pass
    if (a.counters[4] == 0) return;
    if (blockIdx.x == 0 && tid == 0) atomicAdd(&a.counters[3], 1ull);
  }
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const cint* plan = as_const(a.plan);
  const cint* offs = plan + a.off_offs;
  const cint* poffs = plan + a.off_poffs;
  const int bh = plan[a.off_items + 2 * wg];
  int packed = plan[a.off_items + 2 * wg + 1];
  if (packed & kTailFlag) {                     // workgroup-uniform
    tail_pack<DP, MEASURE, FP8>(a, bh, packed & 0xffff, (float*)smem);
    return;
  }
  // part `part` of split row group `split` (-1: a whole row group)
  int split = -1, part = 0;
  if (packed & kSplitFlag) {
    split = (packed & ~kSplitFlag) >> 3;
    part = packed & 7;
    packed = plan[a.off_splits + 2 * split + 1];
  }
  const int i = packed >> 16, t = packed & 0xffff;
  const int o_i = offs[i], n_i = offs[i + 1] - o_i;
  const int row0 = t * WG_ROWS + wave * 32;     // first row of this wave in partition i
  const bool live = row0 < n_i;                 // wave-uniform
  const int myrow = row0 + l32;
  const cint* rinfo = plan + a.off_rows + 4 * i;
  const int e0 = rinfo[0], nf = rinfo[1], nr = rinfo[2];
  // this workgroup's share of the row's fresh blocks [f_lo, f_hi) and reused states
  // [r_lo, r_hi): all of them, or for part p of a split group of np parts the p-th of np
  // consecutive shares of each list ([p n / np, (p + 1) n / np))
  const int np = split < 0 ? 1 : a.split_parts;
  const int f_lo = part * nf / np, f_hi = (part + 1) * nf / np;
  const int r_lo = part * nr / np, r_hi = (part + 1) * nr / np;
  const cint* ent = plan + a.off_ent;
  const float sc = a.scale_log2;
  const float inv_sc = 1.0f / sc;
  const int paddr = partner_addr();
  const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};

  // Q fragment (B operand of S^T = K Q^T): lane holds 8 dims of query row l%32 per chunk
  bf16x8 qf[NKC];
  {
    const uint16_t* Q = (const uint16_t*)a.q + head_base(a, bh);
    const bool ok = myrow < n_i;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const int d0 = kc * 16 + h32 * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ok && d0 < a.D) v = ld16(Q + (size_t)(o_i + myrow) * a.ld + d0);
      qf[kc] = as_bf16x8(v);
    }
  }

  // running merge of the row (base-2 units); its d tiles dt >= AF in LDS between block ends,
  // 4-float chunk q of d tile dt for lane l at ((dt - AF) * 4 + q) * 64 + l (the wave's own
  // region: no barrier)
  f32x16 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = (f32x16){};
  float m_row = kNegInf, l_row = 0.f;
  f32x4* const acc_lds = (f32x4*)(smem + TILE_ELEMS) +
                         (size_t)__builtin_amdgcn_readfirstlane(wave) * (64 * (NDT - AF) * 4);
  auto acc_put = [&](const f32x16 (&v)[NDT]) {
#pragma unroll
    for (int dt = AF; dt < NDT; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        acc_lds[((dt - AF) * 4 + q) * 64 + lane] =
            (f32x4){v[dt][4 * q], v[dt][4 * q + 1], v[dt][4 * q + 2], v[dt][4 * q + 3]};
  };
  auto acc_get = [&](f32x16 (&v)[NDT]) {
#pragma unroll
    for (int dt = AF; dt < NDT; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 w = acc_lds[((dt - AF) * 4 + q) * 64 + lane];
#pragma unroll
        for (int x = 0; x < 4; ++x) v[dt][4 * q + x] = w[x];
      }
  };
  if (AF < NDT && live) acc_put(acc);

  const size_t slot_elems = (size_t)a.slot_rows * DP;
  typename CacheElem<FP8>::type* cache_o = (typename CacheElem<FP8>::type*)a.cache_o;
  const uint16_t* Kg = (const uint16_t*)a.k + head_base(a, bh);
  const uint16_t* VTg = (const uint16_t*)a.vt + (size_t)bh * DP * a.kt_pad;

  // the threads' byte offsets in a tile's loads, the same for every tile: K chunk m is key
  // row c / (DP / 8) of the tile, dims d8 .. d8 + 7 (the last 8 dims of the head for the
  // chunks past D); V^T chunk m is dim c / (KT / 8), keys k8 .. k8 + 7 (c = tid + 256 m)
  const char* const k_end = (const char*)a.k + (size_t)a.B * a.sB * 2;
  uint32_t kbyte[CHK], vbyte[CHV];
#pragma unroll
  for (int m = 0; m < CHK; ++m) {
    const int c = tid + 256 * m;
    kbyte[m] = ((uint32_t)(c / (DP / 8)) * (uint32_t)a.ld + (uint32_t)min((c % (DP / 8)) * 8, a.D - 8)) * 2u;
  }
#pragma unroll
  for (int m = 0; m < CHV; ++m) {
    const int c = tid + 256 * m;
    vbyte[m] = ((uint32_t)(c / (KT / 8)) * (uint32_t)a.kt_pad + (uint32_t)(c % (KT / 8)) * 8u) * 2u;
  }

  // ---------------- fresh blocks ----------------
  for (int e = f_lo; e < f_hi; ++e) {
    const int j = ent[2 * (e0 + e)], slot = ent[2 * (e0 + e) + 1];
    const int o_j = offs[j], n_j = offs[j + 1] - o_j, po_j = poffs[j];
    const int ntile = (n_j + KT - 1) / KT;

    f32x16 bacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) bacc[dt] = (f32x16){};
    // reference: the cached lse (fixed) or the running maximum
    float m_b = FIXED && live
        ? a.cache_lse[((size_t)bh * a.num_slots + slot) * a.slot_rows + myrow] * kLog2e - kRefHeadroom
        : kNegInf;
    float l_b = 0.f;                  // this lane's partial sum (16 of the 32 keys)
    float thr = kNegInf;              // rescale threshold: (m_b + slack) / (tau log2 e)

    // a tile's loads: buffer loads from a resource based at the tile's first key (K: its row,
    // V^T: its column; wave-uniform) at the thread's fixed byte offset.  K rows past the block
    // are read as they stand (the next partition's) or, past the end of K, as zeros, and their
    // scores are masked.
    u32x4 pk[CHK], pv[CHV];
    auto fetch = [&](int kt) {
      const char* Kt = (const char*)(Kg + (size_t)(o_j + kt * KT) * a.ld);
      const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(Kt, (uint64_t)(k_end - Kt));
      const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(VTg + po_j + kt * KT, ~0ull);
#pragma unroll
      for (int m = 0; m < CHK; ++m) pk[m] = buf16(rk, kbyte[m]);
#pragma unroll
      for (int m = 0; m < CHV; ++m) pv[m] = buf16(rv, vbyte[m]);
    };
    fetch(0);
    for (int kt = 0; kt < ntile; ++kt) {
      __syncthreads();   // everyone is done reading the previous tile
#pragma unroll
      for (int m = 0; m < CHK; ++m) {
        const int c = tid + 256 * m;
        st16(&sK[(c / (DP / 8)) * LDK + (c % (DP / 8)) * 8], pk[m]);
      }
#pragma unroll
      for (int m = 0; m < CHV; ++m) {
        const int c = tid + 256 * m;
        st16(&sV[(c / (KT / 8)) * LDV + (c % (KT / 8)) * 8], pv[m]);
      }
      __syncthreads();
      if (kt + 1 < ntile) fetch(kt + 1);
      if (!live) continue;

      // fragment reads from LDS: with AHEAD (DP = 64, where the registers allow it) the next
      // half's K fragments are read as soon as this half's QK MFMAs are issued, and this
      // half's V^T fragments before its softmax, so that the MFMAs seldom wait for the LDS;
      // otherwise each fragment is read where it is used
      auto k_frag = [&](int ks, int kc) {
        return as_bf16x8(ld16(&sK[(ks * 32 + key_of_row(l32)) * LDK + kc * 16 + h32 * 8]));
      };
      auto v_frag = [&](int ks, int dt, int c) {
        return as_f16x8(ld16(&sV[(dt * 32 + l32) * LDV + ks * 32 + c * 16 + h32 * 8]));
      };
      bf16x8 kcur[NKC], knext[NKC];
      if constexpr (AHEAD) {
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) kcur[kc] = k_frag(0, kc);
      }
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int kbase = kt * KT + ks * 32;   // first key of this half (partition-relative)
        if (kbase >= n_j) break;
        // S^T = K Q^T over this 32-key half
        f32x16 s = (f32x16){};
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(AHEAD ? kcur[kc] : k_frag(ks, kc), qf[kc],
                                                      s, 0, 0, 0);
        f16x8 vfr[NDT][2];
        if constexpr (AHEAD) {
          if (ks + 1 < NKS) {
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) knext[kc] = k_frag(ks + 1, kc);
          }
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int c = 0; c < 2; ++c) vfr[dt][c] = v_frag(ks, dt, c);
        }
        if (kbase + 32 > n_j) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kbase + 16 * (r >> 3) + 8 * h32 + (r & 7);
            if (key >= n_j) s[r] = kNegInf;
          }
        }
        if constexpr (!FIXED) {
          // this lane's max over its 16 keys against the rescale threshold (in score units);
          // the query's exact max over both lanes is formed only when a rescale is due
          float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
          for (int r = 3; r < 16; r += 2) mx = fmaxf(fmaxf(mx, s[r]), s[r + 1 < 16 ? r + 1 : r]);
          if (__any(mx > thr)) {
            const float m_new = fmaxf(m_b, max_halves(mx, paddr) * sc);
            const float alpha = fast_exp2(m_b - m_new);
            m_b = m_new;
            thr = (m_new + kRescaleSlack) * inv_sc;
            l_b *= alpha;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) bacc[dt] *= alpha;
          }
        }
        f16x8 pf[2];
#pragma unroll
        for (int r = 0; r < 16; ++r)
          pf[r >> 3][r & 7] = (_Float16)fast_exp2(__builtin_fmaf(s[r], sc, -m_b));
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int q2 = 0; q2 < 4; ++q2) {
            const f16x2 pair = {pf[c][2 * q2], pf[c][2 * q2 + 1]};
            l_b = __builtin_amdgcn_fdot2(pair, ones, l_b, false);
          }
        // O^T += V^T P^T
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int c = 0; c < 2; ++c)
            bacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(AHEAD ? vfr[dt][c] : v_frag(ks, dt, c),
                                                              pf[c], bacc[dt], 0, 0, 0);
        if constexpr (AHEAD) {
#pragma unroll
          for (int kc = 0; kc < NKC; ++kc) kcur[kc] = knext[kc];
        }
      }
    }
    if (!live) continue;
    if constexpr (FIXED) {
      const float lsum = sum_halves(l_b, paddr);
      if (__any(myrow < n_i && !(lsum >= kRefLo && lsum <= kRefHi)) && lane == 0)
        atomicOr(&a.counters[4], 1ull);
    }

    if (AF < NDT) acc_get(acc);
    block_end<NDT, MEASURE, FP8>(a, bacc, m_b, l_b, paddr, (size_t)bh * a.num_slots + slot, row0, myrow,
                   cache_o + ((size_t)bh * a.num_slots + slot) * slot_elems + (size_t)row0 * DP,
                   acc, m_row, l_row, j == i, n_i, i, bh);
    if (AF < NDT) acc_put(acc);
  }
  if (!live) return;
  if (AF < NDT) acc_get(acc);

  reuse_fold<DP, FP8, 1>(a, bh, row0, e0, nf + r_lo, nf + r_hi, acc, m_row, l_row);
  if (split < 0) {
    finish_rows<DP>(a, bh, o_i, n_i, row0, nf, nr, acc, m_row, l_row);
    return;
  }
  // a split part: the partial merge of its rows to the workspace, for merge_splits
  float* ws = a.split_ws + (size_t)(split * a.split_parts + part) * (2 + NDT * 16) * 256 + tid;
  ws[0] = m_row;
  ws[256] = l_row;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int x = 0; x < 16; ++x) ws[(2 + dt * 16 + x) * 256] = acc[dt][x];
}

// The parts of each split row group merged (DiTango, "State-Centric Parallel Runtime /
// Composizione dello Stato": partial attention states combine through their log-sum-exp in
// any grouping; here as partial merges of the rows: part p's weighted by 2^(m_p - m), m the
// largest, summed in the order of the parts, whichever finished first), then the rows written
// as finish_rows does for a whole group.  One wave per (split group, 32-row sub-tile):
// workgroup 4 s + w takes the values wave w of each part's workgroup left, thread for
// thread.  In the conditional second pass it runs only if the first pass rejected a
// reference.
template <int DP>
__global__ __launch_bounds__(64) void merge_splits(StepArgs a) {
  constexpr int NDT = DP / 32;
  constexpr int W = 2 + NDT * 16;
  const int wave = blockIdx.x % kWaves, tid = wave * 64 + (int)threadIdx.x;
  if (a.fixup && a.counters[4] == 0) return;
  const int s = blockIdx.x / kWaves;
  const cint* plan = as_const(a.plan);
  const int bh = plan[a.off_splits + 2 * s], packed = plan[a.off_splits + 2 * s + 1];
  const int i = packed >> 16, t = packed & 0xffff;
  const cint* offs = plan + a.off_offs;
  const int o_i = offs[i], n_i = offs[i + 1] - o_i;
  const int row0 = t * kWaves * 32 + wave * 32;
  if (row0 >= n_i) return;                      // wave-uniform: no rows here
  const cint* rinfo = plan + a.off_rows + 4 * i;
  const int np = a.split_parts;
  const float* w0 = a.split_ws + (size_t)s * np * W * 256 + tid;
  float m = kNegInf;
  for (int p = 0; p < np; ++p) m = fmaxf(m, w0[(size_t)p * W * 256]);
  float l = 0.f;
  f32x16 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = (f32x16){};
  for (int p = 0; p < np; ++p) {
    const float* w = w0 + (size_t)p * W * 256;
    const float mp = w[0];
    const float f = mp == kNegInf ? 0.f : fast_exp2(mp - m);
    l = __builtin_fmaf(w[256], f, l);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int x = 0; x < 16; ++x)
        acc[dt][x] = __builtin_fmaf(w[(2 + dt * 16 + x) * 256], f, acc[dt][x]);
  }
  finish_rows<DP>(a, bh, o_i, n_i, row0, rinfo[1], rinfo[2], acc, m, l);
}

// ------------------------------------------------------------------------------------------
// f32 step: one lane per query row, plain fp32 arithmetic (D <= 64, multiple of 4)
// grid: num_tiles * B*H workgroups of 64 lanes
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(64) void step_f32(StepArgs a) {
  constexpr int DP = 64;
  constexpr int KB = 64;                       // keys staged per LDS round
  __shared__ __attribute__((aligned(16))) float sK[KB][DP];
  __shared__ __attribute__((aligned(16))) float sV[KB][DP];
  const int lane = threadIdx.x;
  const int wg = blockIdx.x;
  const int bh = wg / a.num_tiles, tix = wg - bh * a.num_tiles;
  const int* plan = a.plan;
  const int* offs = plan + a.off_offs;
  const int packed = plan[a.off_tiles + tix];
  const int i = packed >> 16, t = packed & 0xffff;
  const int o_i = offs[i], n_i = offs[i + 1] - o_i;
  const int r = t * kF32Rows + lane;
  const bool ok = r < n_i;
  const int D = a.D;
  const int* rinfo = plan + a.off_rows + 4 * i;
  const int e0 = rinfo[0], nf = rinfo[1], nr = rinfo[2];
  const int* ent = plan + a.off_ent;
  const size_t bhN = (size_t)bh * a.N;
  const size_t hb = head_base(a, bh);
  const int ld = a.ld;
  const float* Q = (const float*)a.q + hb;
  const float* K = (const float*)a.k + hb;
  const float* V = (const float*)a.v + hb;
  float* cache_o = (float*)a.cache_o;

  float q[DP];
#pragma unroll
  for (int d = 0; d < DP; ++d) q[d] = (ok && d < D) ? Q[(size_t)(o_i + r) * ld + d] : 0.f;
  float acc[DP];
#pragma unroll
  for (int d = 0; d < DP; ++d) acc[d] = 0.f;
  float m_row = kNegInf, l_row = 0.f;
  const float sc = a.scale_log2;

  for (int e = 0; e < nf; ++e) {
    const int j = ent[2 * (e0 + e)], slot = ent[2 * (e0 + e) + 1];
    const int o_j = offs[j], n_j = offs[j + 1] - o_j;
    float b[DP];
#pragma unroll
    for (int d = 0; d < DP; ++d) b[d] = 0.f;
    float m_b = kNegInf, l_b = 0.f;
    for (int c0 = 0; c0 < n_j; c0 += KB) {
      __syncthreads();
      const int key = c0 + lane;
#pragma unroll 4
      for (int d = 0; d < DP; ++d) {
        const bool kv = key < n_j && d < D;
        sK[lane][d] = kv ? K[(size_t)(o_j + key) * ld + d] : 0.f;
        sV[lane][d] = kv ? V[(size_t)(o_j + key) * ld + d] : 0.f;
      }
      __syncthreads();
      const int nk = n_j - c0 < KB ? n_j - c0 : KB;
      for (int c = 0; c < nk; ++c) {
        // dot product as four interleaved partial sums of 16 terms
        float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
        for (int d = 0; d < DP; d += 4) {
          p0 = __builtin_fmaf(q[d], sK[c][d], p0);
          p1 = __builtin_fmaf(q[d + 1], sK[c][d + 1], p1);
          p2 = __builtin_fmaf(q[d + 2], sK[c][d + 2], p2);
          p3 = __builtin_fmaf(q[d + 3], sK[c][d + 3], p3);
        }
        const float z = ((p0 + p1) + (p2 + p3)) * sc;
        const float m_new = fmaxf(m_b, z);
        const float alpha = fast_exp2(m_b - m_new);
        const float p = fast_exp2(z - m_new);
        l_b = l_b * alpha + p;
#pragma unroll
        for (int d = 0; d < DP; ++d) b[d] = __builtin_fmaf(p, sV[c][d], b[d] * alpha);
        m_b = m_new;
      }
    }
    const float lse2 = m_b + fast_log2(l_b);
    const size_t base = (size_t)bh * a.num_slots + slot;
    float* dst = cache_o + base * (size_t)DP * a.slot_rows;
    if (j == i && a.delta_part) {
      // planner measurement: squared change of the cached diagonal state, per 32-row half
      float sq = 0.f;
#pragma unroll
      for (int d = 0; d < DP; ++d) {
        const float df = b[d] / l_b - dst[(size_t)d * a.slot_rows + r];
        if (ok && d < D) sq = __builtin_fmaf(df, df, sq);
      }
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) sq += __shfl_xor(sq, off);
      if ((lane & 31) == 0 && t * kF32Rows + lane < n_i)
        a.delta_part[((size_t)bh * a.P + i) * a.delta_stride + ((t * kF32Rows + lane) >> 5)] = sq;
    }
#pragma unroll
    for (int d = 0; d < DP; ++d) {
      b[d] = b[d] / l_b;
      dst[(size_t)d * a.slot_rows + r] = b[d];
    }
    a.cache_lse[base * a.slot_rows + r] = lse2 * kLn2;
    const float mn = fmaxf(m_row, lse2);
    const float fa = fast_exp2(m_row - mn), fb = fast_exp2(lse2 - mn);
#pragma unroll
    for (int d = 0; d < DP; ++d) acc[d] = acc[d] * fa + b[d] * fb;
    l_row = l_row * fa + fb;
    m_row = mn;
  }
  for (int e = nf; e < nf + nr; ++e) {
    const int slot = ent[2 * (e0 + e) + 1];
    const size_t base = (size_t)bh * a.num_slots + slot;
    const float lse2 = a.cache_lse[base * a.slot_rows + r] * kLog2e;
    const float* src = cache_o + base * (size_t)DP * a.slot_rows;
    const float mn = fmaxf(m_row, lse2);
    const float fa = fast_exp2(m_row - mn), fb = fast_exp2(lse2 - mn);
#pragma unroll
    for (int d = 0; d < DP; ++d) acc[d] = acc[d] * fa + src[(size_t)d * a.slot_rows + r] * fb;
    l_row = l_row * fa + fb;
    m_row = mn;
  }
  if (ok) {
    float* orow = (float*)a.out + hb + (size_t)(o_i + r) * ld;
#pragma unroll
    for (int d = 0; d < DP; ++d)
      if (d < D) orow[d] = acc[d] / l_row;
    if (a.lse_out) a.lse_out[bhN + o_i + r] = (m_row + fast_log2(l_row)) * kLn2;
  }
  if (t == 0 && lane == 0) {
    atomicAdd(&a.counters[0], (unsigned long long)nf);
    atomicAdd(&a.counters[1], (unsigned long long)nr);
  }
}

// ------------------------------------------------------------------------------------------
// read one cache slot into row-major f32 (n_i x D) and lse (n_i)
// ------------------------------------------------------------------------------------------
__global__ void read_slot(StepArgs a, int bh, int slot, int n_i, float* o_out, float* lse_out,
                          int esz) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int D = a.D, DP = a.DP;
  const size_t base = (size_t)bh * a.num_slots + slot;
  if (idx < n_i) lse_out[idx] = a.cache_lse[base * a.slot_rows + idx];
  if (idx >= n_i * D) return;
  const int row = idx / D, d = idx - row * D;
  float val;
  if (esz != 4) {
    // fragment order: sub-tile row/32, d tile d/32, lane (d%32/4 odd ? 32 : 0) + row%32,
    // value 4*(d%32/8) + d%4
    const int u = row >> 5, l32 = row & 31, dt = d >> 5, dd = d & 31;
    const int h = (dd >> 2) & 1, reg = 4 * (dd >> 3) + (dd & 3);
    const int lane = h * 32 + l32;
    const size_t off = base * (size_t)a.slot_rows * DP + (size_t)u * 32 * DP + dt * 1024 + lane * 16;
    if (esz == 2) {
      val = (float)__builtin_bit_cast(__bf16, ((const uint16_t*)a.cache_o)[off + reg]);
    } else {
      float v[16];
      fp8_unpack16(ld16((const uint8_t*)a.cache_o + off), v);
      val = v[reg];
    }
  } else {
    const float* src = (const float*)a.cache_o + base * (size_t)DP * a.slot_rows;
    val = src[(size_t)d * a.slot_rows + row];
  }
  o_out[idx] = val;
}

// ------------------------------------------------------------------------------------------
// planner reductions (one workgroup per query partition i, fixed summation order)
// ------------------------------------------------------------------------------------------
// Sum of 256 per-thread doubles, tree order fixed; the result is in red[0].
// Snapshot of the diagonal slots' cached O before a measuring step: one workgroup per
// (partition i, b*h) copies the slot of block (i, i) (found among row i's fresh entries:
// the diagonal block is always fresh) in 16-byte words.
__global__ __launch_bounds__(256) void snapshot_diag(StepArgs a, int slot_bytes) {
  const int i = blockIdx.x, bh = blockIdx.y;
  const cint* plan = as_const(a.plan);
  const cint* rinfo = plan + a.off_rows + 4 * i;
  const cint* ent = plan + a.off_ent;
  const int e0 = rinfo[0], nf = rinfo[1];
  int slot = -1;
  for (int e = 0; e < nf; ++e)
    if (ent[2 * (e0 + e)] == i) slot = ent[2 * (e0 + e) + 1];
  if (slot < 0) return;
  const u32x4* src = (const u32x4*)((const uint8_t*)a.cache_o +
                                    ((size_t)bh * a.num_slots + slot) * (size_t)slot_bytes);
  u32x4* dst = (u32x4*)((uint8_t*)a.diag_snap + ((size_t)bh * a.P + i) * (size_t)slot_bytes);
  for (int w = threadIdx.x; w < slot_bytes / 16; w += 256) dst[w] = src[w];
}

// The change of the diagonal states a measuring step wrote, against the snapshot of them taken
// before the step: per (b, h, i, 32-row sub-tile) the sum over rows < n_i and d < D of
// (new - old)^2, summed in block_end's order (per lane over d tiles and accumulator rows, then
// over the wave), into delta_part.  Grid (P, B*H); one wave per sub-tile.
template <int DP, bool FP8>
__global__ __launch_bounds__(256) void diag_change(StepArgs a) {
  constexpr int NDT = DP / 32;
  typedef typename CacheElem<FP8>::type CT;
  const int i = blockIdx.x, bh = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h32 = lane >> 5, l32 = lane & 31;
  const cint* plan = as_const(a.plan);
  const cint* offs = plan + a.off_offs;
  const cint* rinfo = plan + a.off_rows + 4 * i;
  const cint* ent = plan + a.off_ent;
  const int n_i = offs[i + 1] - offs[i];
  const int e0 = rinfo[0], nf = rinfo[1];
  int slot = -1;
  for (int e = 0; e < nf; ++e)
    if (ent[2 * (e0 + e)] == i) slot = ent[2 * (e0 + e) + 1];
  if (slot < 0) return;
  const size_t slot_elems = (size_t)a.slot_rows * DP;
  const CT* nw = (const CT*)a.cache_o + ((size_t)bh * a.num_slots + slot) * slot_elems;
  const CT* od = (const CT*)a.diag_snap + ((size_t)bh * a.P + i) * slot_elems;
  const int S = (n_i + 31) / 32;
  for (int t = wave; t < S; t += kWaves) {               // wave-uniform
    const int myrow = t * 32 + l32;
    const CT* nt = nw + (size_t)t * 32 * DP;
    const CT* ot = od + (size_t)t * 32 * DP;
    float sq = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      float nv[16], ov[16];
      if constexpr (FP8) {
        fp8_unpack16(ld16(nt + dt * 1024 + lane * 16), nv);
        fp8_unpack16(ld16(ot + dt * 1024 + lane * 16), ov);
      } else {
        const bf16x8 n0 = as_bf16x8(ld16(nt + dt * 1024 + lane * 16));
        const bf16x8 n1 = as_bf16x8(ld16(nt + dt * 1024 + lane * 16 + 8));
        const bf16x8 p0 = as_bf16x8(ld16(ot + dt * 1024 + lane * 16));
        const bf16x8 p1 = as_bf16x8(ld16(ot + dt * 1024 + lane * 16 + 8));
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          nv[r] = (float)n0[r]; nv[r + 8] = (float)n1[r];
          ov[r] = (float)p0[r]; ov[r + 8] = (float)p1[r];
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // accumulator row r of d tile dt holds d = dt*32 + 8*(r/4) + 4*h32 + r%4
        const int d = dt * 32 + 8 * (r >> 2) + 4 * h32 + (r & 3);
        const float df = nv[r] - ov[r];
        if (myrow < n_i && d < a.D) sq = __builtin_fmaf(df, df, sq);
      }
    }
    sq = wave_sum(sq);
    if (lane == 0) a.delta_part[((size_t)bh * a.P + i) * a.delta_stride + t] = sq;
  }
}

__device__ __forceinline__ void block_sum(double* red, double x) {
  red[threadIdx.x] = x;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if ((int)threadIdx.x < st) red[threadIdx.x] += red[threadIdx.x + st];
    __syncthreads();
  }
}

// delta[i] = sqrt(sum of the diagonal block's squared changes / (B H n_i D))
__global__ __launch_bounds__(256) void planner_delta(StepArgs a, float* delta) {
  __shared__ double red[256];
  const int i = blockIdx.x;
  const cint* offs = as_const(a.plan) + a.off_offs;
  const int n_i = offs[i + 1] - offs[i];
  const int S = (n_i + 31) / 32;               // sub-tiles with rows
  const int BH = a.B * a.H;
  double acc = 0.0;
  for (int k = threadIdx.x; k < BH * S; k += 256) {
    const int bh = k / S, sub = k - bh * S;
    acc += (double)a.delta_part[((size_t)bh * a.P + i) * a.delta_stride + sub];
  }
  block_sum(red, acc);
  if (threadIdx.x == 0) delta[i] = (float)sqrt(red[0] / ((double)BH * n_i * a.D));
}

// Importance, stage 1: workgroup (c, i) takes chunk c of the C chunks of the (b, h, r) rows
// of partition i and writes, for every block j of row i's lists (an anchor plan lists every
// active block), the chunk's sum of exp(lse_ij[r] - L_i[r]) to part[(i C + c) P + j] (0 for
// the other j).
__global__ __launch_bounds__(256) void planner_weights_part(StepArgs a, float* part, int C) {
  constexpr int JB = 32;                        // blocks per pass
  __shared__ double red[256];
  const int c = blockIdx.x, i = blockIdx.y, tid = threadIdx.x;
  const cint* plan = as_const(a.plan);
  const cint* offs = plan + a.off_offs;
  const int n_i = offs[i + 1] - offs[i];
  const cint* rinfo = plan + a.off_rows + 4 * i;
  const int e0 = rinfo[0], nb = rinfo[1] + rinfo[2];
  const cint* ent = plan + a.off_ent;
  const int rows = a.B * a.H * n_i;
  const int q0 = (int)((long long)rows * c / C), q1 = (int)((long long)rows * (c + 1) / C);
  float* out = part + ((size_t)i * C + c) * a.P;
  for (int j = tid; j < a.P; j += 256) out[j] = 0.f;
  __syncthreads();
  for (int c0 = 0; c0 < nb; c0 += JB) {
    double accj[JB];
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) accj[jj] = 0.0;
    for (int q = q0 + tid; q < q1; q += 256) {
      const int bh = q / n_i, r = q - bh * n_i;
      const float* lrow = a.cache_lse + (size_t)bh * a.num_slots * a.slot_rows + r;
      float mx = kNegInf;
      for (int e = 0; e < nb; ++e) mx = fmaxf(mx, lrow[(size_t)ent[2 * (e0 + e) + 1] * a.slot_rows]);
      float ssum = 0.f;
      for (int e = 0; e < nb; ++e) ssum += expf(lrow[(size_t)ent[2 * (e0 + e) + 1] * a.slot_rows] - mx);
      const float L = mx + logf(ssum);
#pragma unroll
      for (int jj = 0; jj < JB; ++jj)
        if (c0 + jj < nb)
          accj[jj] += (double)expf(lrow[(size_t)ent[2 * (e0 + c0 + jj) + 1] * a.slot_rows] - L);
    }
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
      if (c0 + jj < nb) {                       // workgroup-uniform
        block_sum(red, accj[jj]);
        if (tid == 0) out[ent[2 * (e0 + c0 + jj)]] = (float)red[0];
        __syncthreads();
      }
    }
  }
}

// Importance, stage 2: w[i P + j] = (sum over chunks c, ascending, of part) / (B H n_i).
__global__ __launch_bounds__(256) void planner_weights_sum(StepArgs a, const float* part, int C,
                                                           float* w) {
  const int i = blockIdx.x;
  const cint* offs = as_const(a.plan) + a.off_offs;
  const double rows = (double)a.B * a.H * (offs[i + 1] - offs[i]);
  for (int j = threadIdx.x; j < a.P; j += 256) {
    double t = 0.0;
    for (int c = 0; c < C; ++c) t += (double)part[((size_t)i * C + c) * a.P + j];
    w[(size_t)i * a.P + j] = (float)(t / rows);
  }
}

// ------------------------------------------------------------------------------------------
// group composition: merge cached states of one row partition into one slot
// workgroup (k, u, bh): 32-row sub-tile u of job k = {n_i, dst slot, first source, number
// of sources}; sources are slots (the destination among them).  Per row: L = log sum_s
// exp(lse_s), O = sum_s exp(lse_s - L) O_s in f32, stored rounded to the cache precision.
// Every lse is read before the destination's is written, and each O element is read and
// written by the same thread.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void merge_slots(StepArgs a, const int32_t* jobs,
                                                   const int32_t* srcs, int esz) {
  __shared__ float Ls[32];
  const int k = blockIdx.x, u = blockIdx.y, bh = blockIdx.z, tid = threadIdx.x;
  const int n_i = jobs[4 * k], dst = jobs[4 * k + 1], s0 = jobs[4 * k + 2], ns = jobs[4 * k + 3];
  if (u * 32 >= n_i) return;                    // workgroup-uniform
  const int DP = a.DP;
  const size_t slot_elems = (size_t)a.slot_rows * DP;
  auto lse_of = [&](int slot, int row) {
    return a.cache_lse[((size_t)bh * a.num_slots + slot) * a.slot_rows + row];
  };
  if (tid < 32) {
    const int row = u * 32 + tid;
    float L = kNegInf;
    if (row < n_i) {
      float mx = kNegInf;
      for (int q = 0; q < ns; ++q) mx = fmaxf(mx, lse_of(srcs[s0 + q], row));
      float sum = 0.f;
      for (int q = 0; q < ns; ++q) sum += expf(lse_of(srcs[s0 + q], row) - mx);
      L = mx + logf(sum);
    }
    Ls[tid] = L;
  }
  __syncthreads();
  if (esz == 1) {
    uint8_t* cache = (uint8_t*)a.cache_o;
    // fp8: 16-byte chunk c = one lane's 16 values of d tile c/64 (lane c%64, row lane%32)
    for (int c = tid; c < DP * 2; c += 256) {
      const int dt = c >> 6, lane = c & 63;
      const int r = lane & 31, row = u * 32 + r;
      if (row >= n_i) continue;
      const size_t off = (size_t)u * 32 * DP + dt * 1024 + lane * 16;
      f32x16 acc = (f32x16){};
      for (int q = 0; q < ns; ++q) {
        const int sl = srcs[s0 + q];
        const float w = expf(lse_of(sl, row) - Ls[r]);
        float v[16];
        fp8_unpack16(ld16(cache + ((size_t)bh * a.num_slots + sl) * slot_elems + off), v);
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = __builtin_fmaf(w, v[e], acc[e]);
      }
      st16(cache + ((size_t)bh * a.num_slots + dst) * slot_elems + off, fp8_pack16(acc));
    }
  } else if (esz == 2) {
    uint16_t* cache = (uint16_t*)a.cache_o;
    // the sub-tile is [DP/32 d tiles][64 lanes][16 values]; 16-byte chunk c: d tile c/128,
    // lane (c/2)%64, half c%2; lane l holds query row l%32
    for (int c = tid; c < DP * 4; c += 256) {
      const int dt = c >> 7, lane = (c >> 1) & 63, half = c & 1;
      const int r = lane & 31, row = u * 32 + r;
      if (row >= n_i) continue;
      const size_t off = (size_t)u * 32 * DP + dt * 1024 + lane * 16 + half * 8;
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int q = 0; q < ns; ++q) {
        const int sl = srcs[s0 + q];
        const float w = expf(lse_of(sl, row) - Ls[r]);
        const bf16x8 v = as_bf16x8(ld16(cache + ((size_t)bh * a.num_slots + sl) * slot_elems + off));
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(w, (float)v[e], acc[e]);
      }
      u32x4 o;
      uint16_t* op = (uint16_t*)&o;
#pragma unroll
      for (int e = 0; e < 8; ++e) op[e] = __builtin_bit_cast(uint16_t, (__bf16)acc[e]);
      st16(cache + ((size_t)bh * a.num_slots + dst) * slot_elems + off, o);
    }
  } else {
    float* cache = (float*)a.cache_o;
    for (int e = tid; e < DP * 32; e += 256) {
      const int d = e >> 5, r = e & 31, row = u * 32 + r;
      if (row >= n_i) continue;
      float acc = 0.f;
      for (int q = 0; q < ns; ++q) {
        const int sl = srcs[s0 + q];
        acc = __builtin_fmaf(expf(lse_of(sl, row) - Ls[r]),
                             cache[((size_t)bh * a.num_slots + sl) * slot_elems + (size_t)d * a.slot_rows + row],
                             acc);
      }
      cache[((size_t)bh * a.num_slots + dst) * slot_elems + (size_t)d * a.slot_rows + row] = acc;
    }
  }
  __syncthreads();
  if (tid < 32 && u * 32 + tid < n_i)
    a.cache_lse[((size_t)bh * a.num_slots + dst) * a.slot_rows + u * 32 + tid] = Ls[tid];
}

// ------------------------------------------------------------------------------------------
// cache compaction / expansion: copy stored states between two slot tables
// workgroup (k, bh): pair k = {new slot, old slot} of map; the slot's lse row (slot_rows f32)
// and its O (o_slot_bytes, a multiple of 16) go from the old buffer to the new one.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void remap_slots(const float* old_lse, const uint8_t* old_o,
                                                   float* new_lse, uint8_t* new_o,
                                                   const int32_t* map, int old_slots,
                                                   int new_slots, int slot_rows,
                                                   long long o_slot_bytes) {
  const int k = blockIdx.x, bh = blockIdx.y;
  const int ns = map[2 * k], os = map[2 * k + 1];
  const float* ls = old_lse + ((size_t)bh * old_slots + os) * slot_rows;
  float* ld = new_lse + ((size_t)bh * new_slots + ns) * slot_rows;
  for (int r = threadIdx.x; r < slot_rows; r += 256) ld[r] = ls[r];
  const u32x4* src = (const u32x4*)(old_o + ((size_t)bh * old_slots + os) * (size_t)o_slot_bytes);
  u32x4* dst = (u32x4*)(new_o + ((size_t)bh * new_slots + ns) * (size_t)o_slot_bytes);
  for (long long w = threadIdx.x; w < o_slot_bytes / 16; w += 256) dst[w] = src[w];
}

}  // namespace

hipError_t launch_remap_slots(const float* old_lse, const void* old_o, float* new_lse,
                              void* new_o, const int32_t* map, int npairs, int bhs,
                              int old_slots, int new_slots, int slot_rows,
                              size_t o_slot_bytes, hipStream_t s) {
  if (npairs == 0) return hipSuccess;
  hipLaunchKernelGGL(remap_slots, dim3(npairs, bhs), dim3(256), 0, s, old_lse,
                     (const uint8_t*)old_o, new_lse, (uint8_t*)new_o, map, old_slots,
                     new_slots, slot_rows, (long long)o_slot_bytes);
  return hipGetLastError();
}

// Scratch of the allocation-free step, for callers that cannot allocate (graph capture, tight
// serving loops): each GPU the library runs on holds its own copy until the process ends.
// Every call on a GPU shares it, so calls that overlap on one GPU race.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

hipError_t static_scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_zero_counters(unsigned long long* counters, int n, hipStream_t s) {
  hipLaunchKernelGGL(zero_u64, dim3((n + 63) / 64), dim3(64), 0, s, counters, n);
  return hipGetLastError();
}

hipError_t launch_transpose_v(const StepArgs& a, hipStream_t s) {
  dim3 grid(a.kt_pad / kKeyTile, a.B * a.H);
  hipLaunchKernelGGL(transpose_v, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_step_bf16(const StepArgs& args, hipStream_t s) {
  const int G = args.num_items;
  StepArgs a = args;
  a.fixup = 0;
  // a measuring step takes the fixed-reference pass only with the snapshot of the old diagonal
  // states (a second pass would otherwise measure against the first pass's writes)
  const int m = a.delta_part != nullptr ? 1 : 0, f = a.cache_fp8 ? 2 : 0;
  const bool fixed = a.fixed_ref && (!m || a.diag_snap);
#define DITA_MERGE_SPLITS(DPV)                                                                   \
  if (a.num_splits > 0) hipLaunchKernelGGL((merge_splits<DPV>), dim3(a.num_splits * kWaves), dim3(64), 0, s, a);
#define DITA_LAUNCH_BF16(DPV)                                                                    \
  if (fixed) {                                                                                   \
    switch (m | f) {                                                                             \
      case 0: hipLaunchKernelGGL((step_bf16<DPV, false, false, true>), dim3(G), dim3(256), 0, s, a); break; \
      case 1: hipLaunchKernelGGL((step_bf16<DPV, true, false, true>), dim3(G), dim3(256), 0, s, a); break;  \
      case 2: hipLaunchKernelGGL((step_bf16<DPV, false, true, true>), dim3(G), dim3(256), 0, s, a); break;  \
      default: hipLaunchKernelGGL((step_bf16<DPV, true, true, true>), dim3(G), dim3(256), 0, s, a); break;  \
    }                                                                                            \
    DITA_MERGE_SPLITS(DPV)                                                                       \
    a.fixup = 1;                                                                                 \
  }                                                                                              \
  switch (m | f) {                                                                               \
    case 0: hipLaunchKernelGGL((step_bf16<DPV, false, false, false>), dim3(G), dim3(256), 0, s, a); break; \
    case 1: hipLaunchKernelGGL((step_bf16<DPV, true, false, false>), dim3(G), dim3(256), 0, s, a); break;  \
    case 2: hipLaunchKernelGGL((step_bf16<DPV, false, true, false>), dim3(G), dim3(256), 0, s, a); break;  \
    default: hipLaunchKernelGGL((step_bf16<DPV, true, true, false>), dim3(G), dim3(256), 0, s, a); break;  \
  }                                                                                              \
  DITA_MERGE_SPLITS(DPV)
  switch (a.DP) {
    case 64: DITA_LAUNCH_BF16(64) break;
    case 96: DITA_LAUNCH_BF16(96) break;
    case 128: DITA_LAUNCH_BF16(128) break;
    default: return hipErrorInvalidValue;
  }
#undef DITA_LAUNCH_BF16
#undef DITA_MERGE_SPLITS
  return hipGetLastError();
}

hipError_t launch_step_f32(const StepArgs& a, hipStream_t s) {
  const int G = a.num_tiles * a.B * a.H;
  hipLaunchKernelGGL(step_f32, dim3(G), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_snapshot_diag(const StepArgs& a, hipStream_t s) {
  const int slot_bytes = a.slot_rows * a.DP * (a.cache_fp8 ? 1 : 2);
  hipLaunchKernelGGL(snapshot_diag, dim3(a.P, a.B * a.H), dim3(256), 0, s, a, slot_bytes);
  return hipGetLastError();
}

hipError_t launch_diag_change(const StepArgs& a, hipStream_t s) {
  const dim3 grid(a.P, a.B * a.H);
#define DITA_LAUNCH_DC(DPV)                                                                      \
  if (a.cache_fp8) hipLaunchKernelGGL((diag_change<DPV, true>), grid, dim3(256), 0, s, a);       \
  else hipLaunchKernelGGL((diag_change<DPV, false>), grid, dim3(256), 0, s, a);
  switch (a.DP) {
    case 64: DITA_LAUNCH_DC(64) break;
    case 96: DITA_LAUNCH_DC(96) break;
    case 128: DITA_LAUNCH_DC(128) break;
    default: return hipErrorInvalidValue;
  }
#undef DITA_LAUNCH_DC
  return hipGetLastError();
}

hipError_t launch_planner_delta(const StepArgs& a, float* delta, hipStream_t s) {
  hipLaunchKernelGGL(planner_delta, dim3(a.P), dim3(256), 0, s, a, delta);
  return hipGetLastError();
}

hipError_t launch_planner_weights(const StepArgs& a, float* w, float* part, hipStream_t s) {
  const int C = planner_chunks(a.P);
  hipLaunchKernelGGL(planner_weights_part, dim3(C, a.P), dim3(256), 0, s, a, part, C);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(planner_weights_sum, dim3(a.P), dim3(256), 0, s, a, part, C, w);
  return hipGetLastError();
}

hipError_t launch_merge_slots(const StepArgs& a, const int32_t* jobs, const int32_t* srcs,
                              int njobs, int cache_esz, hipStream_t s) {
  hipLaunchKernelGGL(merge_slots, dim3(njobs, a.slot_rows / 32, a.B * a.H), dim3(256), 0, s, a,
                     jobs, srcs, cache_esz);
  return hipGetLastError();
}

hipError_t launch_read_slot(const StepArgs& a, int bh, int slot, int n_i, float* o_out,
                            float* lse_out, int cache_esz, hipStream_t s) {
  const int n = n_i * a.D;
  hipLaunchKernelGGL(read_slot, dim3((n + 255) / 256), dim3(256), 0, s, a, bh, slot, n_i,
                     o_out, lse_out, cache_esz);
  return hipGetLastError();
}

}  // namespace dita
