// attn_common.h -- CDNA4 (gfx950) building blocks of the attention kernels.
//
// Matrix cores: v_mfma_f32_32x32x16_bf16, one wave64.  Operand lane layout
// (lane l, element e of the 8 bf16 an operand register holds, h = l / 32):
//   A (32 x 16):  row l % 32, k = 8h + e
//   B (16 x 32):  col l % 32, k = 8h + e
//   C (32 x 32):  16 floats, element v at col l % 32, row 8(v/4) + 4h + v%4
// A contraction may permute k freely as long as A and B agree.  The kernels
// keep score tiles transposed (keys in the rows of C) so that each lane owns
// one query row (forward, dQ) or one key column (dK/dV): its interval runs
// are loop-invariant registers and row statistics need only one exchange with
// lane l ^ 32.  A score block in C layout feeds the next contraction as a B
// operand directly when the other operand lists its k in the order
//   pi(8h + e) = 4h + e (e < 4),  8 + 4h + (e - 4) (e >= 4)
// within each 16-wide k chunk.
//
// ds_read_b64_tr_b16 (gfx950): in each 16-lane group, lane r supplies the
// address of 4 bf16; lane i receives element i % 4 of the 4-bf16 words of
// lanes 4e + i / 4, e = 0..3.  Pointing lane r at row kb + r / 4, column
// nb + 4 (r % 4) of a row-major [k][n] LDS tile gives lane i the column
// nb + i at rows kb..kb+3: a transposed read, so V, Q, dO and K stay
// row-major in LDS and still serve as k-major MFMA operands.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cm {
namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ uint4 as_u4(const bf16x8& v) { return __builtin_bit_cast(uint4, v); }

__device__ __forceinline__ bf16x8 lds_read_b128(const uint16_t* p) {
  return as_bf16x8(*reinterpret_cast<const uint4*>(p));
}

// transposed read of 4 bf16 (see header comment)
__device__ __forceinline__ bf16x4 lds_read_tr4(const uint16_t* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 cat4(const bf16x4& a, const bf16x4& b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ float wave_xor32(float x) { return __shfl_xor(x, 32, 64); }

// max(x, x of lane l ^ 32) without a trip through LDS: gfx950's
// v_permlane32_swap exchanges the upper 32 lanes of one register with the
// lower 32 of another, so swapping two copies of x leaves x's lower half in
// both halves of one and its upper half in both halves of the other.  (The
// wait states cover a vector write of the copies just before.)
__device__ __forceinline__ float wave_xor32_max(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return fmaxf(a, b);
}

__device__ __forceinline__ uint32_t uniform(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }

// Swizzled row-major LDS tile of D bf16 columns (no padding).  The 16-byte
// chunk c of row r lives at chunk c ^ f(r).  f makes both access patterns the
// kernels use conflict-free on 64 four-byte banks: 16 consecutive rows read at
// one chunk (MFMA operand rows, ds_read_b128), and 4 consecutive rows (from a
// multiple of 4) read across 4 consecutive chunks (ds_read_b64_tr_b16).
template <int D>
__device__ __forceinline__ int swz_f(int row) {
  static_assert(D == 64 || D == 128, "head dim");
  return (D == 128) ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}
template <int D>
__device__ __forceinline__ int swz(int row, int col) {
  return row * D + ((((col >> 3) ^ swz_f<D>(row)) << 3) | (col & 7));
}

typedef __attribute__((address_space(3))) void lds_void_t;

// Buffer resource over one (sample, head) slice of a [.., N, stride_n] bf16
// tensor: rows at or past N read as zero (hardware range check).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slice_rsrc(const void* base, int N, int64_t sn, int D) {
  const uint32_t bytes = uint32_t(((int64_t(N) - 1) * sn + D) * 2);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}

// Asynchronous copy of a BR x D bf16 tile from global memory straight into a
// swizzled LDS tile (buffer_load ... lds, 16 bytes per lane).  Each wave
// instruction fills 1 KiB of LDS contiguously (lane l at +16 l), so every lane
// fetches the global chunk that belongs at its LDS slot.  The NW waves of the
// work-group share the tile.  Completion: s_waitcnt vmcnt + a barrier.
template <int D, int BR, int NW>
struct TileDma {
  static constexpr int BLOCKS = BR * D * 2 / 1024;
  static constexpr int PER_WAVE = BLOCKS / NW;
  static_assert(BLOCKS % NW == 0, "tile split");
  uint32_t voff[PER_WAVE];
  int wave;
  __device__ void init(int wave_, int lane, int64_t sn) {
    wave = wave_;
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int p = (wave * PER_WAVE + j) * 512 + lane * 8;  // element index in the LDS tile
      const int row = p / D, pc = (p % D) >> 3;
      const int lc = pc ^ swz_f<D>(row);
      voff[j] = uint32_t((int64_t(row) * sn + lc * 8) * 2);
    }
  }
  // row0_bytes: byte offset of the tile's first row in the slice (wave-uniform)
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, uint16_t* lds_tile, uint32_t row0_bytes) const {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(lds_tile + (wave * PER_WAVE + j) * 512), 16, voff[j],
                                               row0_bytes, 0, 0);
#endif
  }
};

// One wave copies 64 consecutive floats (starting `first_bytes` into the
// buffer) straight into LDS.  (The LDS-copy builtins exist only in the device
// pass; the host pass, which only needs the kernels' launch stubs, skips them.)
__device__ __forceinline__ void dma_row_floats(__amdgpu_buffer_rsrc_t rs, float* lds, int lane, uint32_t first_bytes) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)lds, 4, uint32_t(lane * 4), first_bytes, 0, 0);
#endif
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Per-lane byte offsets of the LDS operand reads inside one swizzled BR x D
// tile (row-major, D bf16 per row).
//   row[m]     : MFMA A-operand rows, ds_read_b128 of row (lane % 32), d chunk
//                16 m + 8 h; the second 32-row block adds 32 D * 2 bytes.
//   tr(db, hf) : transposed reads for the k-major operand of d block db: the
//                address lane (g, gi) supplies for rows 8 hf + 4 (g / 2) +
//                gi / 4, columns 32 db + 16 (g % 2) + 4 (gi % 4); each further
//                16-row chunk adds 16 D * 2 bytes.
// The swizzle only depends on the low four row bits, so the row-block and
// 16-row offsets are immediates of the LDS instructions.
// With COMPACT, the second half (hf = 1, eight rows further) is formed on the
// fly: it differs from the first by a per-lane constant, since the swizzle of
// rows 8..15 flips chunk bit 1, which for these lanes is g % 2 whatever db
// is.  That saves D / 32 registers for one add per transposed pair.
template <int D, bool COMPACT>
struct LdsOffsets {
  uint32_t row[D / 16];
  uint32_t tr0[D / 32];
  uint32_t tr1[COMPACT ? 1 : D / 32];
  __device__ __forceinline__ void init(int lane) {
    const int h = lane >> 5, lr = lane & 31, g = lane >> 4, gi = lane & 15;
#pragma unroll
    for (int m = 0; m < D / 16; ++m) row[m] = uint32_t(swz<D>(lr, 16 * m + 8 * h)) * 2u;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      tr0[db] = uint32_t(swz<D>(4 * (g >> 1) + (gi >> 2), db * 32 + 16 * (g & 1) + 4 * (gi & 3))) * 2u;
      if (!COMPACT) tr1[db] = uint32_t(swz<D>(8 + 4 * (g >> 1) + (gi >> 2), db * 32 + 16 * (g & 1) + 4 * (gi & 3))) * 2u;
    }
    if (COMPACT) tr1[0] = uint32_t(swz<D>(8 + 4 * (g >> 1) + (gi >> 2), 16 * (g & 1) + 4 * (gi & 3))) * 2u - tr0[0];
  }
  __device__ __forceinline__ uint32_t tr(int db, int hf) const {
    if (!hf) return tr0[db];
    return COMPACT ? tr0[db] + tr1[0] : tr1[COMPACT ? 0 : db];
  }
};

__device__ __forceinline__ bf16x8 lds_b128_at(const char* p) {
  return as_bf16x8(*reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ bf16x8 lds_tr8_at(const char* p0, const char* p1) {
  return cat4(lds_read_tr4(reinterpret_cast<const uint16_t*>(p0)), lds_read_tr4(reinterpret_cast<const uint16_t*>(p1)));
}

// Scheduling-group masks (AMDGPU sched_group_barrier).
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// A run of NM MFMAs whose A operands come from LDS: read(i) returns operand i
// and mma(i, a) issues MFMA i (MPO matrix instructions per operand).  Operand
// reads run G MFMAs ahead of their use (a register pipeline of G + 1
// operands), and the scheduling groups keep that order: G reads, then (MFMA,
// next read) pairs.  RPO = LDS instructions per operand (1 for ds_read_b128,
// 2 for a pair of transposed reads).
template <int NM, int G, int RPO, int MPO = 1, class Read, class Mma>
__device__ __forceinline__ void mfma_stream(Read&& read, Mma&& mma) {
  constexpr int G0 = G < NM ? G : NM;
  bf16x8 op[NM];
#pragma unroll
  for (int i = 0; i < G0; ++i) op[i] = read(i);
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    if (i + G < NM) op[i + G] = read(i + G);
    mma(i, op[i]);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, RPO * G0, 0);
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, MPO, 0);
    if (i + G < NM) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, RPO, 0);
  }
}

// Precision of the probabilities (P) and score gradients (dS) where they
// enter a matrix product as bf16 operands (PV forward; dV, dK, dQ backward).
//   kPrecBf16 (the default): rounded to bf16 once, as tiled attention usually
//     does: a relative error of up to 2^-9 per element.
//   kPrecSplit: x = hi + lo with hi = bf16(x) and lo = bf16(x - hi), two
//     matrix instructions per operand pair, about 2^-17 relative error: the
//     products then carry the fp32 values up to accumulation order.
constexpr int kPrecBf16 = 0;
constexpr int kPrecSplit = 1;

__device__ __forceinline__ __bf16 bf16_lo(float x, __bf16 hi) { return (__bf16)(x - float(hi)); }

// Offset, inside a 64-wide tile, of element v of 32-block blk of a score
// tile in C layout, for the lane half h = 0 (add 4h for the other half).
__host__ __device__ __forceinline__ constexpr uint32_t elem_offset(int blk, int v) {
  return uint32_t(blk * 32 + (v >> 2) * 8 + (v & 3));
}

// Partial-tile visibility checks.  A lane's interval data are loop-invariant
// registers (LaneRuns); `base` is the tile's first index plus 4h, so element
// e of the tile sits at index j = base + elem_offset(e).
//   kCheckRunBits (the default): each visible run [start, start + length) is
//     turned into a range of the lane's element numbers with a few endpoint
//     compares per run and tile (elements ordered by index, so a run covers
//     a contiguous range of them), the ranges are OR-ed into one 32-bit word,
//     and each element then costs one bit extract and one bit select.  The
//     per-element work no longer grows with the number of runs.
//   kCheckUnsigned: the visible runs as (start, length); j is visible when
//     (j - start) <u length for some run: one subtraction (hoisted) and one
//     compare per run and element (CompileMask paper summary, section 3.3.2).
//   kCheckOrdinaryMasked: the ablation the paper summary compares against
//     (section 4.4, Table 3): the complement of the visible runs as masked
//     intervals [lo, hi), and j is masked when lo <= j and j < hi for some
//     interval: two compares and their conjunction per interval.
// Invisible elements become `fill` (-inf for scores before a softmax, 0 for
// probabilities).
constexpr int kCheckRunBits = 0;
constexpr int kCheckOrdinaryMasked = 1;
constexpr int kCheckUnsigned = 3;

// How many of a lane's 32 tile elements have an index below x.  The
// elements sit at base + 8k + i (k = 0..7, i = 0..3), so with y = x - base
// clamped to [0, 64] the count is 4 floor(y / 8) + min(y mod 8, 4).  (x and
// base are at most N + 63 < 2^31, so the signed difference is exact.)
__host__ __device__ __forceinline__ uint32_t elems_below(uint32_t x, uint32_t base) {
  const int y = min(max(int(x - base), 0), 64);
  return uint32_t(((y >> 3) << 2) + min(y & 7, 4));
}

// Bits [lo, hi) of a 32-bit word, 0 <= lo <= hi <= 32.
__host__ __device__ __forceinline__ uint32_t bit_range(uint32_t lo, uint32_t hi) {
  const uint32_t w = hi - lo;
  return w >= 32u ? 0xFFFFFFFFu : (((1u << w) - 1u) << (lo & 31u));
}

// Bits of the lane's elements inside the run [start, start + len).
__host__ __device__ __forceinline__ uint32_t run_bits(uint32_t start, uint32_t len, uint32_t base) {
  return bit_range(elems_below(start, base), elems_below(start + len, base));
}

// Keep the elements whose bit is set, the others become fill: per element a
// sign-extended one-bit extract (all ones or zero) and a bit select.
__device__ __forceinline__ void apply_bits(f32x16 (&s)[2], uint32_t bits, float fill) {
  const uint32_t f = __builtin_bit_cast(uint32_t, fill);
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const uint32_t m = uint32_t(int32_t(bits << (31 - e)) >> 31);
    // (the element goes through a scalar first: clang's __builtin_bit_cast
    // applied directly to a vector subscript reads element 0)
    const float sv = s[e >> 4][e & 15];
    const uint32_t x = __builtin_bit_cast(uint32_t, sv);
    s[e >> 4][e & 15] = __builtin_bit_cast(float, (x & m) | (f & ~m));
  }
}

// A lane's first MAXR visible runs as (start, length); absent runs are
// (0, 0) and only follow present ones.
template <int MAXR>
struct LaneRuns {
  uint32_t a[MAXR], b[MAXR];
};

// Check against the first NR runs held in registers (NR <= MAXR; every run
// of the tile's rows or columns is among them).
template <int NR, int CHK, int MAXR>
__device__ __forceinline__ void mask_runs(f32x16 (&s)[2], uint32_t base, const LaneRuns<MAXR>& lr, float fill) {
  if (CHK == kCheckRunBits) {
    uint32_t bits = 0;
#pragma unroll
    for (int r = 0; r < NR; ++r) bits |= run_bits(lr.a[r], lr.b[r], base);
    apply_bits(s, bits, fill);
  } else if (CHK == kCheckUnsigned) {
    uint32_t off[NR > 0 ? NR : 1];
#pragma unroll
    for (int r = 0; r < NR; ++r) off[r] = base - lr.a[r];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        bool vis = false;
#pragma unroll
        for (int r = 0; r < NR; ++r) vis = vis | (off[r] + elem_offset(blk, v) < lr.b[r]);
        s[blk][v] = vis ? s[blk][v] : fill;
      }
    }
  } else {
    // the masked intervals: before each present run, and after the last one
    // (formed here, per tile: the empty asm keeps the compiler from hoisting
    // them, and everything derived from them, out of the tile loop)
    uint32_t lo[NR + 1], hi[NR + 1], prev = 0;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      uint32_t st = lr.a[r], len = lr.b[r];
      asm volatile("" : "+v"(st), "+v"(len));
      const bool present = len > 0;
      lo[r] = present ? prev : 0u;
      hi[r] = present ? st : 0u;
      prev = present ? st + len : prev;
    }
    lo[NR] = prev;
    hi[NR] = 0xFFFFFFFFu;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const uint32_t j = base + elem_offset(blk, v);
        bool masked = false;
#pragma unroll
        for (int k = 0; k <= NR; ++k) masked = masked || ((j >= lo[k]) && (j < hi[k]));
        s[blk][v] = masked ? fill : s[blk][v];
      }
    }
  }
}

// Run-bitmask word from runs read from memory, four runs per round with
// their loads issued before any is used (entries between the lane's own run
// count and nr are zero-length padding).
__device__ __forceinline__ uint32_t runs_bits_mem(uint32_t base, const uint2* runs, int nr, bool valid);

// Same check with the runs read from memory (rows or columns with more runs
// than the register copy holds).
template <int CHK>
__device__ __forceinline__ void mask_runs_mem(f32x16 (&s)[2], uint32_t base, const uint2* runs, int nr, bool valid,
                                              float fill) {
  uint32_t bits = 0;
  if (CHK == kCheckRunBits) {
    bits = runs_bits_mem(base, runs, nr, valid);
  } else if (CHK == kCheckUnsigned) {
    for (int r = 0; r < nr; ++r) {
      const uint2 rr = valid ? runs[r] : make_uint2(0u, 0u);
      const uint32_t off = base - rr.x, len = rr.y - rr.x;
#pragma unroll
      for (int e = 0; e < 32; ++e) bits |= uint32_t(off + elem_offset(e >> 4, e & 15) < len) << e;
    }
  } else {
    uint32_t masked = 0, prev = 0;
    for (int r = 0; r < nr; ++r) {
      const uint2 rr = valid ? runs[r] : make_uint2(0u, 0u);
      if (rr.y > rr.x) {
        uint32_t jb = base;
        asm volatile("" : "+v"(jb));  // indices formed per run, not hoisted
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          const uint32_t j = jb + elem_offset(e >> 4, e & 15);
          masked |= uint32_t((j >= prev) && (j < rr.x)) << e;
        }
        prev = rr.y;
      }
    }
#pragma unroll
    for (int e = 0; e < 32; ++e) masked |= uint32_t(base + elem_offset(e >> 4, e & 15) >= prev) << e;
    bits = ~masked;
  }
  if (CHK == kCheckRunBits) {
    apply_bits(s, bits, fill);
    return;
  }
#pragma unroll
  for (int e = 0; e < 32; ++e) s[e >> 4][e & 15] = ((bits >> e) & 1u) ? s[e >> 4][e & 15] : fill;
}

// Dispatch on the tile's run maximum (wave-uniform): up to MAXR runs come
// from registers, more from memory.
template <int CHK, int MAXR>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[2], uint32_t base, int nr, const LaneRuns<MAXR>& lr,
                                          const uint2* runs, bool valid, float fill) {
  static_assert(MAXR == 1 || MAXR == 2 || MAXR == 4, "register copy holds 1, 2 or 4 runs");
  switch (nr) {
    case 0: mask_runs<0, CHK>(s, base, lr, fill); break;
    case 1: mask_runs<1, CHK>(s, base, lr, fill); break;
    case 2:
      if (MAXR >= 2) { mask_runs<(MAXR >= 2 ? 2 : 0), CHK>(s, base, lr, fill); break; }
      [[fallthrough]];
    case 3:
      if (MAXR >= 3) { mask_runs<(MAXR >= 3 ? 3 : 0), CHK>(s, base, lr, fill); break; }
      [[fallthrough]];
    case 4:
      if (MAXR >= 4) { mask_runs<(MAXR >= 4 ? 4 : 0), CHK>(s, base, lr, fill); break; }
      [[fallthrough]];
    default: mask_runs_mem<CHK>(s, base, runs, nr, valid, fill); break;
  }
}

// The run-bitmask visibility word of one tile on its own, before any score
// exists: the kernels test it across the wave first (a tile no row or column
// of the wave sees is skipped; one that all of them see entirely needs no
// select).  Same dispatch on the tile's run maximum as mask_tile.
template <int NR, int MAXR>
__device__ __forceinline__ uint32_t runs_bits(uint32_t base, const LaneRuns<MAXR>& lr) {
  uint32_t bits = 0;
#pragma unroll
  for (int r = 0; r < NR; ++r) bits |= run_bits(lr.a[r], lr.b[r], base);
  return bits;
}

__device__ __forceinline__ uint32_t runs_bits_mem(uint32_t base, const uint2* runs, int nr, bool valid) {
  uint32_t bits = 0;
  for (int r = 0; r < nr; r += 4) {
    uint2 rr[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) rr[t] = (valid && r + t < nr) ? runs[r + t] : make_uint2(0u, 0u);
#pragma unroll
    for (int t = 0; t < 4; ++t) bits |= run_bits(rr[t].x, rr[t].y - rr[t].x, base);
  }
  return bits;
}

template <int MAXR>
__device__ __forceinline__ uint32_t tile_bits(uint32_t base, int nr, const LaneRuns<MAXR>& lr, const uint2* runs,
                                              bool valid) {
  static_assert(MAXR == 1 || MAXR == 2 || MAXR == 4, "register copy holds 1, 2 or 4 runs");
  switch (nr) {
    case 0: return 0u;
    case 1: return runs_bits<1>(base, lr);
    case 2:
      if (MAXR >= 2) return runs_bits<(MAXR >= 2 ? 2 : 1)>(base, lr);
      [[fallthrough]];
    case 3:
      if (MAXR >= 3) return runs_bits<(MAXR >= 3 ? 3 : 1)>(base, lr);
      [[fallthrough]];
    case 4:
      if (MAXR >= 4) return runs_bits<(MAXR >= 4 ? 4 : 1)>(base, lr);
      [[fallthrough]];
    default: return runs_bits_mem(base, runs, nr, valid);
  }
}

// What a wave does with a masked tile under the run bitmask: skip it (no
// lane sees any element), run it unmasked (every lane sees every element),
// or select per element.
struct WaveTile {
  uint32_t bits;
  bool skip, select;
  __device__ __forceinline__ void init(uint32_t b) {
    bits = b;
    skip = !__any(b != 0u);
    select = !__all(b == 0xFFFFFFFFu);
  }
};

// The lane's first MAXR runs from its interval-table row (the first `nr`
// entries, nr being the tile's run maximum) or, on the maskless causal path,
// the single run given as [start, end).
template <int MAXR>
__device__ __forceinline__ LaneRuns<MAXR> load_runs(bool causal, uint2 causal_run, const uint2* row, int nr,
                                                    bool valid) {
  LaneRuns<MAXR> lr;
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    uint2 v = make_uint2(0u, 0u);
    if (causal) { if (r == 0) v = causal_run; }
    else if (r < nr && valid) v = row[r];
    lr.a[r] = v.x;
    lr.b[r] = v.y - v.x;
  }
  return lr;
}

// ------------------------------------------------------------------ predicate baseline
//
// The comparison point the CompileMask pages measure against (paper summary,
// sections 1 and 4.2: FlexAttention-style masking): the mask is a predicate of
// (row i, key j) evaluated element by element inside partial tiles, with the
// inputs it needs (the segment of each token, the references of a segment)
// read from memory at each evaluation.  Families, as the workloads define
// them:
//   causal         j <= i
//   hstu           i < h ? j <= i : (j < h || j == i)
//   shared_prompt  i < P ? j <= i : (j < P || (seg(i) >= 0 && seg(j) == seg(i) && j <= i))
//   retrieval      i < g ? j <= i : (j < g || (seg(i) >= 0 && seg(j) >= 0 &&
//                  ((seg(j) == seg(i) && j <= i) || seg(j) == ref_r(seg(i)) for some r)))
// (at most two references per segment).
constexpr int kCheckPredicate = 2;
enum PredFamily : int { kPredCausal = 0, kPredHstu = 1, kPredSharedPrompt = 2, kPredRetrieval = 3 };

struct PredCtx {
  int32_t family;
  const int32_t* tok_seg;    // [B][N] segment of each token, -1 = none
  const int32_t* scalars;    // [B][n_scalars]; the family's scalar is entry 0
  int32_t n_scalars;
  const int32_t* refs;       // [B][seg_cap][n_refs]
  int32_t seg_cap, n_refs;
  const uint32_t* sample_err;  // [B], from the block-mask build
};

// One sample's view of the predicate inputs.
struct PredSample {
  int32_t family, N, scalar, n_refs;
  bool valid;
  const int32_t* seg;   // [N]
  const int32_t* refs;  // [seg_cap][n_refs]
  __device__ __forceinline__ void init(const PredCtx& c, int b, int N_) {
    family = c.family;
    N = N_;
    n_refs = c.n_refs;
    valid = c.sample_err[b] == 0u;
    scalar = (c.n_scalars > 0) ? c.scalars[size_t(b) * c.n_scalars] : 0;
    seg = c.tok_seg + size_t(b) * N_;
    refs = c.refs ? c.refs + size_t(b) * c.seg_cap * c.n_refs : nullptr;
  }
};

// Visibility of (i, j), both inside [0, N); seg_i / seg_j are seg(i) / seg(j)
// when the caller has them (-2 = read from memory here).
__device__ __forceinline__ bool pred_visible(const PredSample& p, int i, int j, int seg_i, int seg_j = -2) {
  if (!p.valid) return false;
  switch (p.family) {
    case kPredCausal:
      return j <= i;
    case kPredHstu:
      return i < p.scalar ? j <= i : (j < p.scalar || j == i);
    case kPredSharedPrompt: {
      if (i < p.scalar) return j <= i;
      if (j < p.scalar) return true;
      const int si = seg_i == -2 ? p.seg[i] : seg_i;
      return si >= 0 && j <= i && (seg_j == -2 ? p.seg[j] : seg_j) == si;
    }
    default: {  // kPredRetrieval
      if (i < p.scalar) return j <= i;
      if (j < p.scalar) return true;
      const int si = seg_i == -2 ? p.seg[i] : seg_i;
      if (si < 0) return false;
      const int sj = seg_j == -2 ? p.seg[j] : seg_j;
      if (sj < 0) return false;
      if (sj == si) return j <= i;
      for (int r = 0; r < p.n_refs; ++r)
        if (p.refs[si * p.n_refs + r] == sj) return true;
      return false;
    }
  }
}

// The predicate from inputs already in registers: si, sj = seg(i), seg(j);
// r0, r1 = the references of seg(i) (-1 = none; at most two).
__device__ __forceinline__ bool pred_eval(int family, bool valid, int scalar, int i, int j, int si, int sj, int r0,
                                          int r1) {
  const bool causal = j <= i;
  bool vis;
  if (family == kPredCausal) {
    vis = causal;
  } else if (family == kPredHstu) {
    vis = i < scalar ? causal : (j < scalar || j == i);
  } else if (family == kPredSharedPrompt) {
    vis = i < scalar ? causal : (j < scalar || (si >= 0 && sj == si && causal));
  } else {
    const bool seg_ok = si >= 0 && sj >= 0;
    vis = i < scalar ? causal : (j < scalar || (seg_ok && ((sj == si && causal) || sj == r0 || sj == r1)));
  }
  return valid && vis;
}

// Partial-tile check of the predicate baseline.  LANE_IS_ROW: the lane owns
// row `lane_idx` and the tile's elements are keys (forward, dQ); otherwise the
// lane owns key `lane_idx` and the elements are rows (dK/dV).  The per-token
// inputs of the tile's elements are gathered first (independent loads, as a
// tiled predicate kernel loads them for its block), then the predicate is
// evaluated from registers.  Elements past N are invisible.
template <bool LANE_IS_ROW>
__device__ __forceinline__ void mask_pred(f32x16 (&s)[2], uint32_t base, int lane_idx, bool lane_valid,
                                          const PredSample& ps, float fill) {
  const bool segs = ps.family >= kPredSharedPrompt;
  const bool refs = ps.family == kPredRetrieval && ps.n_refs > 0;
  const int seg_lane = (lane_valid && segs) ? ps.seg[lane_idx] : -1;
  int lane_r0 = -1, lane_r1 = -1;
  if (LANE_IS_ROW && refs && seg_lane >= 0) {
    lane_r0 = ps.refs[seg_lane * ps.n_refs];
    if (ps.n_refs > 1) lane_r1 = ps.refs[seg_lane * ps.n_refs + 1];
  }
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {  // one 32-block (16 elements) at a time
    int se[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int x = int(base + elem_offset(blk, v));
      se[v] = (segs && x < ps.N) ? ps.seg[x] : -1;
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int x = int(base + elem_offset(blk, v));
      int r0 = lane_r0, r1 = lane_r1;
      if (!LANE_IS_ROW && refs) {  // the row is the element: its segment's references
        r0 = se[v] >= 0 ? ps.refs[se[v] * ps.n_refs] : -1;
        r1 = (se[v] >= 0 && ps.n_refs > 1) ? ps.refs[se[v] * ps.n_refs + 1] : -1;
      }
      const int i = LANE_IS_ROW ? lane_idx : x, j = LANE_IS_ROW ? x : lane_idx;
      const int si = LANE_IS_ROW ? seg_lane : se[v], sj = LANE_IS_ROW ? se[v] : seg_lane;
      const bool vis = lane_valid && x < ps.N && pred_eval(ps.family, ps.valid, ps.scalar, i, j, si, sj, r0, r1);
      s[blk][v] = vis ? s[blk][v] : fill;
    }
  }
}

// XCD-aware work-group order.  MI355X deals consecutive work-group ids
// round-robin to its 8 XCDs, each with its own L2.  With a 1-D grid of
// tiles * hb work-groups (hb = samples x heads), ids are remapped so that
// every (sample, head) is handled by one XCD (when hb is a multiple of 8):
// the tiles of one head that run at the same time then stream the same
// K/V (or Q/dO) tiles through the same L2.  Each XCD holds hb / 8 heads;
// it deals their tiles either tile by tile (`interleave`: tile k of every
// head, then tile k + 1, ...) or head by head.  Tile k is the k-th in the
// kernel's own order, which puts the longest tiles of lower-triangular masks
// first: interleaving keeps every head's long tiles ahead of every head's
// short ones.  The kernels interleave heads of fewer than kInterleaveBelow
// tiles.  Head by head, an XCD's running work-groups share one head's
// streamed tiles in L2; interleaved, they stream every head's.  Measured on
// MI355X: interleaving 32- and 64-tile heads saves about 5% of each kernel,
// while for 256-tile heads it gains nothing and doubles the forward's and
// dQ's HBM reads.
constexpr int kXcds = 8;
constexpr int kInterleaveBelow = 128;
__device__ __forceinline__ void xcd_coords(int w, int tiles, int hb, bool interleave, int& k, int& bh) {
  if (hb % kXcds == 0) {
    const int xcd = w % kXcds, local = w / kXcds, hpx = hb / kXcds;
    if (interleave) {
      bh = xcd + kXcds * (local % hpx);
      k = local / hpx;
    } else {
      bh = xcd + kXcds * (local / tiles);
      k = local % tiles;
    }
  } else {
    bh = w / tiles;
    k = w % tiles;
  }
}

// Visit the non-empty tiles of one bitmap row (codes 1 full, 2 partial).
// The next bitmap word is loaded while the current one is consumed, so the
// wave does not wait for a memory round trip every 16 tiles.
struct TileIter {
  const uint32_t* words;
  int W, w;
  uint32_t word, pending, ahead;
  __device__ void init(const uint32_t* p, int nwords) {
    words = p; W = nwords; w = -1; word = 0; pending = 0;
    ahead = nwords > 0 ? p[0] : 0u;
  }
  // next non-empty tile; false at the end
  __device__ __forceinline__ bool next(int& tile, int& state) {
    while (pending == 0) {
      if (++w >= W) return false;
      word = uniform(ahead);
      if (w + 1 < W) ahead = words[w + 1];
      pending = (word | (word >> 1)) & 0x55555555u;
    }
    const int bit = __builtin_ctz(pending);
    pending &= pending - 1;
    tile = w * 16 + bit / 2;
    state = (word >> bit) & 3;
    return true;
  }
};

}  // namespace attn
}  // namespace cm
