// attn_dkdv_wide.hip -- the dK/dV kernel with 64 keys per wave.
//
// Same computation as bwd_dkdv_kernel (attn_bwd.hip): per key column, the
// query tiles that the backward Tile-State Bitmap marks non-empty, with the
// column's visible-row runs checked in partial tiles (CompileMask paper
// summary, section 3.3: the backward traverses the mask by key column, with
// its own direction-aligned intervals):
//   S = Q K^T, P = exp(S - lse) (0 where invisible), dV^T += dO^T P,
//   dP = dO V^T, dS = P (dP - D), dK^T += Q^T dS.
//
// Why a second kernel: with 32 keys per wave every Q or dO operand read from
// LDS feeds one matrix instruction, and at one wave per SIMD the LDS
// instruction rate bounds the kernel.  Here a wave owns 64 keys (two 32-key
// blocks), so each operand read feeds two matrix instructions, one per key
// block: half the LDS reads per MFMA.  The price is registers: K of 64 keys
// as a B operand (64 VGPRs) and the dK, dV accumulators (256 AGPRs, written
// by the inline-asm accumulations below; the score blocks live in VGPRs).
// V of the work-group's 256 keys stays in LDS and is read for dP.
//
// A work-group of four waves covers 256 keys: two consecutive key tiles of a
// 128-key backward grid (waves 0-1 the first, 2-3 the second).  It walks the
// query tiles in the union of the two bitmap rows; each wave takes the tile
// state from its own row, and skips a tile that is empty for it.  Each 64-row
// query tile is done in two 32-row halves.
#include <hip/hip_runtime.h>

#include <cstring>

#include "attn_common.h"
#include "internal.h"

namespace cm {
namespace {

using namespace attn;

struct WideParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dO;
  const float* D;        // rowsum(dO * O), [B][H][N]
  const float* lse2;     // lse * log2(e), +inf for rows with no visible key
  uint16_t* dk;
  uint16_t* dv;
  int64_t sb, sh, sn;
  int32_t B, H, N;
  float scale, scale_log2;
  int32_t Tk_b, Wb;      // the backward grid's key tiles (128 keys) and bitmap words per row
  int32_t pairs;         // work-groups per (sample, head): ceil(Tk_b / 2)
  const uint32_t* bbm;
  const uint2* col_iv;
  int32_t K_c;
  const uint32_t* col_tkmax;
};

typedef int i32x4 __attribute__((ext_vector_type(4)));

// dV^T / dK^T accumulation into AGPRs.  The compiler gives all of a
// function's matrix instructions one register form; this file asks for the
// VGPR form (the score blocks feed vector math), so the accumulating
// instructions are written out with AGPR accumulators.  Back-to-back
// accumulation into the same registers needs no wait states; `fresh` adds
// two before an instruction whose operands vector code has just written.
template <bool FRESH>
__device__ __forceinline__ void mfma_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  const i32x4 ai = __builtin_bit_cast(i32x4, a), bi = __builtin_bit_cast(i32x4, b);
  if (FRESH) asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(ai), "v"(bi));
  else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(ai), "v"(bi));
}

constexpr int BQ = 64;     // query rows per bitmap tile (two 32-row halves)
constexpr int KT = 128;    // keys per backward-grid tile
constexpr int MAXRW = 1;   // column runs per key block held in registers
constexpr int RL = 8;      // column runs per key column staged in LDS; more are read from memory

// Bits v of a lane's 16 elements (one 32-row half of a key block) select the
// score; the others become `fill`.
__device__ __forceinline__ void apply_bits16(f32x16& s, uint32_t bits, float fill) {
  const uint32_t f = __builtin_bit_cast(uint32_t, fill);
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const uint32_t m = uint32_t(int32_t(bits << (31 - e)) >> 31);
    const float sv = s[e];
    const uint32_t x = __builtin_bit_cast(uint32_t, sv);
    s[e] = __builtin_bit_cast(float, (x & m) | (f & ~m));
  }
}

// Bits of a column's first NR staged runs (all reads issued before any is
// used; runs past the column's own count are zero-length padding).
template <int NR>
__device__ __forceinline__ uint32_t staged_bits(uint32_t base, const uint2* staged) {
  uint2 rr[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) rr[r] = staged[r * 256];
  uint32_t bits = 0;
#pragma unroll
  for (int r = 0; r < NR; ++r) bits |= run_bits(rr[r].x, rr[r].y - rr[r].x, base);
  return bits;
}

// The visibility word of one key column over a 64-row tile (bit 16 h + v:
// element v of the lane's half h; see elem_offset): from its run in
// registers, from its first RL runs staged in LDS (`staged`: column-major,
// 256 columns per run index), or for wider tiles from memory.
__device__ __forceinline__ uint32_t column_bits(uint32_t base, int nr, const LaneRuns<MAXRW>& lr, const uint2* staged,
                                                const uint2* runs, bool valid) {
  switch (nr) {
    case 0: return 0u;
    case 1: return runs_bits<1>(base, lr);
    case 2: return staged_bits<2>(base, staged);
    case 3: return staged_bits<3>(base, staged);
    case 4: return staged_bits<4>(base, staged);
    case 5: case 6: return staged_bits<6>(base, staged);
    case 7: case 8: return staged_bits<8>(base, staged);
    default: return runs_bits_mem(base, runs, nr, valid);
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_wide_kernel(WideParams p) {
  constexpr int NW = 4;
  constexpr int TILE = BQ * D;                 // bf16 elements of one Q or dO tile
  constexpr int TB = TILE * 2;                 // its bytes
  constexpr int NC = D / 16;                   // 16-wide d chunks (S, dP contractions)
  constexpr int ND = D / 32;                   // 32-row d blocks of dK^T, dV^T
  // V of the work-group's 256 keys (copied once; dP's B operands), and Q and
  // dO tiles in two stages (stage x holds Q then dO) with the tile's lse2 and
  // D rows: tile t + 1 is copied while tile t is computed.
  __shared__ __attribute__((aligned(1024))) uint16_t sV[256 * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sQO[2][2][TILE];
  __shared__ __attribute__((aligned(16))) float sL[2][BQ];
  __shared__ __attribute__((aligned(16))) float sD[2][BQ];
  __shared__ __attribute__((aligned(16))) uint2 sRuns[CAUSAL ? 1 : RL * 256];  // [run][column]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = int(uniform(uint32_t(tid >> 6)));
  const int h = lane >> 5, lk = lane & 31;
  int pr, bh;
  // heads dealt tile by tile on each XCD: every head's longest key tiles
  // (the first ones, seen by the most rows) start first (see
  // dkdv_wide_supported)
  xcd_coords(int(blockIdx.x), p.pairs, p.B * p.H, true, pr, bh);
  const int head = bh % p.H, b = bh / p.H;
  const int N = p.N;
  const int kt = 2 * pr + (wave >> 1);         // this wave's 128-key tile of the backward grid
  const bool tile_ok = kt < p.Tk_b;
  const int key0 = pr * 256 + wave * 64 + lk;  // key block 0 of this lane; block 1 is key0 + 32
  const bool kv0 = key0 < N, kv1 = key0 + 32 < N;
  const size_t base = size_t(b) * p.sb + size_t(head) * p.sh;
  const size_t rbase = (size_t(b) * p.H + head) * N;
  const __amdgpu_buffer_rsrc_t rQ = slice_rsrc(p.q + base, N, p.sn, D);
  const __amdgpu_buffer_rsrc_t rO = slice_rsrc(p.dO + base, N, p.sn, D);
  const __amdgpu_buffer_rsrc_t rL =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p.lse2 + rbase), 0, N * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rDv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p.D + rbase), 0, N * 4, 0x00020000);
  TileDma<D, BQ, NW> dma;
  dma.init(wave, lane, p.sn);
  const uint32_t tile_bytes = uint32_t(BQ * p.sn * 2);
  auto issue = [&](int tile, int bf) {
    dma.issue(rQ, sQO[bf][0], uint32_t(tile) * tile_bytes);
    dma.issue(rO, sQO[bf][1], uint32_t(tile) * tile_bytes);
    if (wave == 0) dma_row_floats(rL, sL[bf], lane, uint32_t(tile * BQ * 4));
    else if (wave == 1) dma_row_floats(rDv, sD[bf], lane, uint32_t(tile * BQ * 4));
  };
  // Transposed reads (ds_read_b64_tr_b16) of d block db: lane (g, gi) points
  // at row 4 (g / 2) + gi / 4, column 32 db + 16 (g % 2) + 4 (gi % 4) of a
  // 16-row chunk; the d block only moves swizzle bits 2-3 of the chunk index,
  // so the offset is T ^ 64 db, and rows 8 further are T ^ 32 + 8 rows.
  const int g = lane >> 4, gi = lane & 15;
  const int trow = 4 * (g >> 1) + (gi >> 2);
  const uint32_t ftr = uint32_t(swz_f<D>(trow));
  const uint32_t tlow = uint32_t(2 * (g & 1) + ((gi >> 1) & 1));
  const uint32_t trx = (uint32_t(trow) * D * 2) | (16u * (tlow ^ (ftr & 3u))) | (8u * uint32_t(gi & 1)) |
                       ((ftr >> 2) << 6);
  // Row reads (ds_read_b128) of row lk, d chunk c (16 c + 8 h): the swizzled
  // 16-byte chunk is (2 c + h) ^ f = 2 (c ^ (f >> 1)) + (h ^ (f & 1)), so the
  // byte offset is X ^ 32 c with one per-lane X (bits 5.. of X's other terms
  // are clear).
  const uint32_t fsw = uint32_t(swz_f<D>(lk));
  const uint32_t rowx = (uint32_t(lk) * D * 2) | (16u * (uint32_t(h) ^ (fsw & 1u))) | ((fsw >> 1) << 5);

  // the work-group's V rows into LDS (rows past N read as zero), once
  {
    const __amdgpu_buffer_rsrc_t rV = slice_rsrc(p.v + base, N, p.sn, D);
    TileDma<D, 256, NW> vdma;
    vdma.init(wave, lane, p.sn);
    vdma.issue(rV, sV, uint32_t(pr) * 256u * uint32_t(p.sn) * 2u);
  }
  // this wave's keys as B operands of S, two 32-key blocks
  bf16x8 kreg[2][NC];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const bool ok = kb ? kv1 : kv0;
    const size_t row = size_t(key0 + 32 * kb) * p.sn;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint4 uk = make_uint4(0, 0, 0, 0);
      if (ok) uk = *reinterpret_cast<const uint4*>(p.k + base + row + 16 * c + 8 * h);
      kreg[kb][c] = as_bf16x8(uk);
    }
  }
  // dP's B operands: V row (wave * 64 + 32 kb + lk), d chunk c, from LDS
  // (same swizzle position as the Q row reads: rowx ^ 32 c)
  const char* sVw = reinterpret_cast<const char*>(sV) + wave * (64 * D * 2);

  // the visible-row runs of this lane's two key columns
  const int nr = CAUSAL ? 1 : (tile_ok ? int(uniform(p.col_tkmax[size_t(b) * p.Tk_b + kt])) : 0);
  auto col_runs = [&](int kb) -> const uint2* {
    const bool ok = kb ? kv1 : kv0;
    int kk = ok ? key0 + 32 * kb : 0;
    asm volatile("" : "+v"(kk));  // formed where used, not kept live (and spilled) across the loop
    return CAUSAL ? nullptr : p.col_iv + (size_t(b) * N + kk) * p.K_c;
  };
  const LaneRuns<MAXRW> lr0 = load_runs<MAXRW>(CAUSAL, make_uint2(uint32_t(key0), uint32_t(N)), col_runs(0), nr, kv0);
  const LaneRuns<MAXRW> lr1 =
      load_runs<MAXRW>(CAUSAL, make_uint2(uint32_t(key0 + 32), uint32_t(N)), col_runs(1), nr, kv1);
  // the first RL runs of both columns staged in LDS for the partial-tile checks
  // (each wave reads back only its own columns)
  const int colx = wave * 64 + lk;  // the lane's column in the work-group (key block 0; block 1 is + 32)
  if (!CAUSAL && nr > 1 && nr <= RL) {
    // staged_bits reads up to the next even count: runs past nr are staged as (0, 0)
    const int nl = min(RL, nr + (nr & 1));
    for (int kb = 0; kb < 2; ++kb) {
      const bool ok = kb ? kv1 : kv0;
      const uint2* src = col_runs(kb);
      for (int r = 0; r < nl; ++r) sRuns[r * 256 + colx + 32 * kb] = (ok && r < nr) ? src[r] : make_uint2(0u, 0u);
    }
  }

  f32x16 adv[ND][2], adk[ND][2];
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) { adv[db][kb] = f32x16{}; adk[db][kb] = f32x16{}; }

  // query tiles: the union of the two key tiles' bitmap rows (causal: from
  // the first row the work-group's first key can see); the wave's own state
  // comes from its own row
  const uint32_t* row0 = p.bbm + (size_t(b) * p.Tk_b + 2 * pr) * p.Wb;
  const bool has1 = 2 * pr + 1 < p.Tk_b;
  const uint32_t* row1 = row0 + p.Wb;
  const int Tq = (N + BQ - 1) / BQ;
  int w = -1, cnext = (pr * 256) / BQ;
  uint32_t word0 = 0, word1 = 0, pending = 0;
  // the next bitmap words, loaded while the current ones are consumed
  uint32_t ahead0 = 0, ahead1 = 0;
  if (!CAUSAL && p.Wb > 0) {
    ahead0 = row0[0];
    ahead1 = has1 ? row1[0] : 0u;
  }
  auto next_tile = [&](int& tile, int& state) -> bool {
    if (CAUSAL) {
      if (cnext >= Tq) return false;
      tile = cnext++;
      const int kfirst = pr * 256 + wave * 64;  // the wave's first key
      const int klast = min(kfirst + 63, N - 1);
      state = (kfirst >= N || tile * BQ + BQ - 1 < kfirst) ? 0 : (tile * BQ >= klast ? 1 : 2);
      return true;
    }
    while (pending == 0) {
      if (++w >= p.Wb) return false;
      word0 = uniform(ahead0);
      word1 = uniform(ahead1);
      if (w + 1 < p.Wb) {
        ahead0 = row0[w + 1];
        ahead1 = has1 ? row1[w + 1] : 0u;
      }
      pending = ((word0 | (word0 >> 1)) | (word1 | (word1 >> 1))) & 0x55555555u;
    }
    const int bit = __builtin_ctz(pending);
    pending &= pending - 1;
    tile = w * 16 + bit / 2;
    state = (((wave >> 1) ? word1 : word0) >> bit) & 3;
    return true;
  };

  int tile = 0, state = 0, buf = 0;
  bool have = next_tile(tile, state);
  if (have) issue(tile, 0);
  const char* lds0 = reinterpret_cast<const char*>(&sQO[0][0][0]);
  while (have) {
    const int ct = tile, cs = state;
    have = next_tile(tile, state);
    wait_vmem();
    __syncthreads();
    if (have) issue(tile, buf ^ 1);
    const char* cur = lds0 + buf * (2 * TB);
    const float* cL = sL[buf];
    const float* cD = sD[buf];
    buf ^= 1;
    if (cs == 0) continue;  // empty for this wave's keys (the other waves' tile)

    // partial and ragged tiles: the visibility words of both key columns,
    // known before the scores; a tile none of the wave's columns sees is
    // skipped, one they all see entirely runs unmasked
    const bool masked = (cs == 2) || ((ct + 1) * BQ > N);
    uint32_t bits0 = 0xFFFFFFFFu, bits1 = 0xFFFFFFFFu;
    bool select = false;
    if (masked) {
      const uint32_t base_q = uint32_t(ct * BQ + 4 * h);
      bits0 = column_bits(base_q, nr, lr0, sRuns + (CAUSAL ? 0 : colx), col_runs(0), kv0);
      bits1 = column_bits(base_q, nr, lr1, sRuns + (CAUSAL ? 0 : colx + 32), col_runs(1), kv1);
      if (!__any((bits0 | bits1) != 0u)) continue;
      select = !__all((bits0 & bits1) == 0xFFFFFFFFu);
    }

#pragma unroll 1
    for (int hf = 0; hf < 2; ++hf) {
      // One stream of operand reads per 32-row half, each read feeding two
      // MFMAs (one per key block), reads running G operands ahead across the
      // four contractions:
      //   steps [0, NC)        S  += Q  K^T   (Q rows, ds_read_b128)
      //   steps [NC, 2 NC)     dP += dO V^T   (dO rows)
      //   steps [T0, T0 + 2ND) dV^T += dO^T P (dO transposed), per 16-row chunk qc
      //   steps [T1, T1 + 2ND) dK^T += Q^T dS (Q transposed)
      // Vector work rides along, spread so that no step carries much more
      // than its two MFMAs can hide:
      //   the probabilities P = exp2(S log2e/sqrt(d) - lse2), eight chunks x
      //     from step NC + SK (late enough for the last S MFMAs to finish);
      //   chunk qc's bf16 P operands (masked in partial tiles), one key block
      //     per step in the two steps before its dV MFMAs (after that step's
      //     probabilities);
      //   dS = P (dP - D) of chunk qc in ND parts from the last dV step of qc
      //     (each chunk has its own P operands and D values, so chunk qc + 1
      //     is prepared while chunk qc's MFMAs still read chunk qc's);
      //   chunk qc's bf16 dS operands just before its dK MFMAs.
      constexpr int T0 = 2 * NC, T1 = T0 + 2 * ND, NOPS = T1 + 2 * ND, G = 4;
      constexpr int SK = NC / 4;  // exp chunks start this many steps after the last S MFMAs
      const char* qh = cur + hf * (32 * D * 2);
      auto rd = [&](int i) -> bf16x8 {
        if (i < T0) return lds_b128_at(qh + (i < NC ? 0 : TB) + (rowx ^ (uint32_t(i % NC) << 5)));
        const int ph = i < T1 ? 0 : 1, j = i - (ph ? T1 : T0), qc = j / ND, db = j % ND;
        const char* t = cur + (ph == 0 ? TB : 0) + (2 * hf + qc) * (16 * D * 2);
        const uint32_t o0 = trx ^ (uint32_t(db) << 6);
        return lds_tr8_at(t + o0, t + ((o0 ^ 32u) + 8u * D * 2u));
      };
      f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
      bf16x8 op[NOPS], vo[NOPS][2];
      auto rdv = [&](int i, int kb) { return lds_b128_at(sVw + kb * (32 * D * 2) + (rowx ^ (uint32_t(i - NC) << 5))); };
      bf16x8 pb[2][2], sb[2];  // pb[qc][kb]
      // lse2 of row group vg, read two steps before its first use (one
      // buffer per row group: with d = 64 the groups follow each other every
      // step); D of chunk qc's two row groups, read when its dV MFMAs start
      float4 lbuf[4], dbuf[2][2];
      auto lse_step = [](int x) { return NC + SK + x * NC / 8; };  // the step of exp chunk x
#pragma unroll
      for (int i = 0; i < G; ++i) {
        op[i] = rd(i);
        if (i >= NC && i < T0) { vo[i][0] = rdv(i, 0); vo[i][1] = rdv(i, 1); }
      }
#pragma unroll
      for (int i = 0; i < NOPS; ++i) {
        if (i >= T1 && (i - T1) % ND == 0) {
          const int qc = (i - T1) / ND;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 8; ++e) sb[kb][e] = (__bf16)dp[kb][8 * qc + e];
        }
        // the step's MFMA for key block kb
        auto mma_kb = [&](int kb) {
          if (i < NC) {
            s[kb] = mfma32(op[i], kreg[kb][i], s[kb]);
          } else if (i < T0) {
            dp[kb] = mfma32(op[i], vo[i][kb], dp[kb]);
          } else if (i < T1) {
            const int qc = (i - T0) / ND, db = (i - T0) % ND;
            if (db == 0 && kb == 0) mfma_acc<true>(adv[db][kb], op[i], pb[qc][kb]);
            else mfma_acc<false>(adv[db][kb], op[i], pb[qc][kb]);
          } else {
            const int db = (i - T1) % ND;
            if (db == 0 && kb == 0) mfma_acc<true>(adk[db][kb], op[i], sb[kb]);
            else mfma_acc<false>(adk[db][kb], op[i], sb[kb]);
          }
        };
        // The vector work sits between and after the step's two MFMAs, so
        // that it issues in the shadow of each of them rather than in that of
        // the second only.
        mma_kb(0);
        __builtin_amdgcn_sched_barrier(0);
        if (i + G < NOPS) {
          op[i + G] = rd(i + G);
          if (i + G >= NC && i + G < T0) { vo[i + G][0] = rdv(i + G, 0); vo[i + G][1] = rdv(i + G, 1); }
        }
#pragma unroll
        for (int vg = 0; vg < 4; ++vg)
          if (i == lse_step(2 * vg) - 2) lbuf[vg] = *reinterpret_cast<const float4*>(cL + hf * 32 + vg * 8 + 4 * h);
        if (i >= T0 && i < T1 && (i - T0) % ND == 0) {
          const int qc = (i - T0) / ND;
          dbuf[qc][0] = *reinterpret_cast<const float4*>(cD + hf * 32 + (2 * qc) * 8 + 4 * h);
          dbuf[qc][1] = *reinterpret_cast<const float4*>(cD + hf * 32 + (2 * qc + 1) * 8 + 4 * h);
        }
        // probability chunks x = 2 vg + kb (row group vg of the half, key block kb)
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          if (i != lse_step(x)) continue;
          const int vg = x >> 1, kb = x & 1;
          const float4 l4 = lbuf[vg];
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            s[kb][4 * vg + e] = __builtin_amdgcn_exp2f(fmaf(s[kb][4 * vg + e], p.scale_log2, -lv[e]));
          // (pins the chunk to this step: instruction selection would
          // otherwise sink it to its first use and pile chunks up there)
          asm volatile("" : "+v"(s[kb]));
        }
        mma_kb(1);
        __builtin_amdgcn_sched_barrier(0);
        // the bf16 P operands of chunk qc, key block kb (elements 8 qc ..
        // 8 qc + 7), masked in partial tiles
#pragma unroll
        for (int qc = 0; qc < 2; ++qc)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            if (i != T0 + qc * ND - 2 + kb) continue;
            if (select) {
              const uint32_t bits = (kb ? bits1 : bits0) >> (16 * hf + 8 * qc);
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const uint32_t m = uint32_t(int32_t(bits << (31 - e)) >> 31);
                const float sv = s[kb][8 * qc + e];
                s[kb][8 * qc + e] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, sv) & m);
              }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) pb[qc][kb][e] = (__bf16)s[kb][8 * qc + e];
            asm volatile("" : "+v"(pb[qc][kb]), "+v"(s[kb]));
          }
        // dS of chunk qc in ND parts (row group 2 qc + part / (ND / 2)), from
        // its last dV step
#pragma unroll
        for (int qc = 0; qc < 2; ++qc)
#pragma unroll
          for (int part = 0; part < ND; ++part) {
            if (i != T0 + qc * ND + ND - 1 + part) continue;
            constexpr int PER = 16 / ND;  // elements per part (of 2 row groups x 2 key blocks x 4)
            const int g = (part * PER) / 8, kb = ((part * PER) / 4) & 1, e0 = (part * PER) % 4;
            const int vg = 2 * qc + g;
            const float4 d4 = dbuf[qc][g];
            const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int k = 0; k < PER; ++k) {
              const int kk = (e0 + k) / 4, e = (e0 + k) % 4;  // (for PER = 8: both key blocks)
              const int kbx = (kb + kk) & 1;
              const int v = 4 * vg + e;
              dp[kbx][v] = s[kbx][v] * (dp[kbx][v] - dv4[e]);
            }
            asm volatile("" : "+v"(dp[0]), "+v"(dp[1]));
          }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  wait_vmem();  // the V copy of a work-group with no query tile is not left in flight

  // the last accumulating instructions must have written their results
  // before the accumulators are read (wait states after the matrix work)
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7");
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) asm volatile("" : "+a"(adv[db][kb]), "+a"(adk[db][kb]));

  // dK = scale dS^T Q and dV, bf16, one key per lane and key block
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = key0 + 32 * kb;
    if (key >= N) continue;
    uint16_t* dKp = p.dk + base + size_t(key) * p.sn;
    uint16_t* dVp = p.dv + base + size_t(key) * p.sn;
#pragma unroll
    for (int db = 0; db < ND; ++db) {
#pragma unroll
      for (int vg = 0; vg < 4; ++vg) {
        bf16x4 k4, v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          k4[e] = (__bf16)(adk[db][kb][vg * 4 + e] * p.scale);
          v4[e] = (__bf16)(adv[db][kb][vg * 4 + e]);
        }
        *reinterpret_cast<bf16x4*>(dKp + db * 32 + vg * 8 + 4 * h) = k4;
        *reinterpret_cast<bf16x4*>(dVp + db * 32 + vg * 8 + 4 * h) = v4;
      }
    }
  }
}

}  // namespace

// Work-group balance decides where the wide kernel pays.  A 256-key
// work-group does the work of two 128-key ones, so the kernel ends later
// when a few key tiles hold much more work than the rest and start late.
// The kernel deals each XCD's heads tile by tile, so all of them start with
// their first key tiles, which the most rows see: a list-schedule model puts
// retrieval4_32k's makespan 1.8% above the balanced one (38% dealt head by
// head: its global prefix, seen by every row, holds up to eight times the
// mean work) and reward_model_32k's 0.9%.  For hstu_4k (N 4096) the model
// puts 256-key work-groups 18% above balanced against 0.2% with 128-key ones,
// yet since the kernel's step schedule was tightened it runs 7% faster there
// all the same (same-box A/B).  Packed batches keep the 32-keys-per-wave
// kernel (hstu_packed_64k: 2% slower with this one), and so do short
// sequences, where a head has only a few work-groups.
bool dkdv_wide_supported(const AttnDims& a, const DescView& dv) {
  return (a.d == 128 || a.d == 64) && dv.bk == KT && dv.bq == BQ && a.check == CM_CHECK_RUN_BITS &&
         a.precision == CM_PRECISION_BF16 && dv.packed == 0 && a.N >= 2048;
}

hipError_t launch_bwd_dkdv_wide(const AttnDims& a, const void* q, const void* k, const void* v, const void* dO,
                                const float* D, const DescView& dv, void* dk, void* dvv, hipStream_t stream) {
  WideParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.dO = static_cast<const uint16_t*>(dO);
  p.D = D;
  p.lse2 = D + size_t(a.B) * a.H * a.N;
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dvv);
  p.sb = a.sb; p.sh = a.sh; p.sn = a.sn;
  p.B = a.B; p.H = a.H; p.N = a.N;
  p.scale = a.scale;
  p.scale_log2 = a.scale * kLog2e;
  p.Tk_b = (a.N + KT - 1) / KT;
  p.Wb = dv.Wb;
  p.pairs = (p.Tk_b + 1) / 2;
  p.bbm = dv.bbm;
  p.col_iv = reinterpret_cast<const uint2*>(dv.col_iv);
  p.K_c = dv.K_c;
  p.col_tkmax = dv.col_tkmax;
  dim3 grid(unsigned(p.pairs) * a.H * a.B);
  const bool c = a.causal != 0;
  if (a.d == 128) {
    if (c) hipLaunchKernelGGL((bwd_dkdv_wide_kernel<128, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((bwd_dkdv_wide_kernel<128, false>), grid, dim3(256), 0, stream, p);
  } else {
    if (c) hipLaunchKernelGGL((bwd_dkdv_wide_kernel<64, true>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((bwd_dkdv_wide_kernel<64, false>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace cm
