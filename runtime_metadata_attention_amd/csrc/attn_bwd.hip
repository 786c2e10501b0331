// attn_bwd.hip -- descriptor-guided attention backward.
//
// Training throughput counts forward plus backward (CompileMask paper summary,
// section 1), and the backward has its own descriptor direction (section 3.3
// "Online Efficient Mask Attention Execution": forward and backward use
// separate rules so that their intervals follow each pass's traversal).
//
// Three kernels, no atomics, deterministic:
//   D    : D[q] = rowsum(dO[q] * O[q]) in fp32.
//   dK/dV: one work-group per key tile (bwd_k keys), looping over the query
//          tiles its backward bitmap row marks non-empty.  Scores are kept
//          with keys in the columns (lane = key), so each lane's column runs
//          (visible query rows) are loop-invariant registers.
//            S = Q K^T, P = exp(S - lse) (masked in partial tiles),
//            dV^T += dO^T P, dP = dO V^T, dS = P (dP - D), dK^T += Q^T dS.
//   dQ   : one work-group per query tile (fwd_q rows) over the forward
//          bitmap row and the row runs (lane = query):
//            S^T = K Q^T, P^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T.
// K^T, V^T of the work-group's own keys (dK/dV) and Q^T, dO^T of its own
// queries (dQ) stay in registers; the streamed tiles are staged in LDS
// row-major and also read transposed (ds_read_b64_tr_b16).
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "attn_common.h"
#include "internal.h"

namespace cm {
namespace {

using namespace attn;

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dO;
  const float* lse;
  const float* D;        // rowsum(dO * O), [B][H][N]
  const float* lse2;     // lse * log2(e), +inf for rows with no visible key, [B][H][N]
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* Dout;
  float* lse2out;
  int64_t sb, sh, sn;
  int32_t B, H, N, d;
  float scale, scale_log2;
  // forward grid (dQ)
  int32_t Tq_f, Tk_f, Wf;
  const uint32_t* fbm;
  const uint2* row_iv;
  int32_t K_r;
  const uint32_t* row_tkmax;
  // backward grid (dK/dV)
  int32_t Tk_b, Tq_b, Wb;
  const uint32_t* bbm;
  const uint2* col_iv;
  int32_t K_c;
  const uint32_t* col_tkmax;
  PredCtx pred;            // predicate baseline (check kCheckPredicate) only
};

constexpr int MAXR = 4;    // column runs held in registers by the dK/dV kernel
constexpr int MAXR_Q = 2;  // row runs held in registers by the dQ kernel (more are read from memory)
constexpr int BQ = 64;  // query rows per step of the dK/dV kernel
constexpr int BN = 64;  // keys per step of the dQ kernel

// ------------------------------------------------------------------ D

// Four lanes per row, each with D / 32 sixteen-byte chunks of O and dO in
// flight (the chunks of one load instruction are 64 contiguous bytes of 16
// rows); two exchanges finish the row sum.  Rows are at most 2^27 (an
// argument check), so the index arithmetic is 32-bit.
template <int D>
__global__ __launch_bounds__(256) void bwd_dot_kernel(BwdParams p) {
  constexpr int LPR = 4;             // lanes per row
  constexpr int CPL = D / 8 / LPR;   // 16-byte chunks per lane
  constexpr int RPB = 256 / LPR;     // rows per block
  const int t = threadIdx.x, j = t % LPR;
  const int row = int(blockIdx.x) * RPB + t / LPR;
  const int total = p.B * p.H * p.N;
  float acc = 0.f;
  if (row < total) {
    const int n = row % p.N, bh = row / p.N;
    const int hh = bh % p.H, bb = bh / p.H;
    const size_t off = size_t(bb) * p.sb + size_t(hh) * p.sh + size_t(n) * p.sn + j * 8;
    uint4 ua[CPL], ub[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      ua[c] = *reinterpret_cast<const uint4*>(p.o + off + c * (LPR * 8));
      ub[c] = *reinterpret_cast<const uint4*>(p.dO + off + c * (LPR * 8));
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const bf16x8 a = as_bf16x8(ua[c]), b = as_bf16x8(ub[c]);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf(float(a[e]), float(b[e]), acc);
    }
  }
  acc += __shfl_xor(acc, 2, 64);
  acc += __shfl_xor(acc, 1, 64);
  if (row < total && j == 0) {
    p.Dout[row] = acc;
    const float x = p.lse[row];
    p.lse2out[row] = (x == -INFINITY) ? INFINITY : x * kLog2e;
  }
}

// ------------------------------------------------------------------ dK / dV

template <int D, int BK, bool CAUSAL, int CHK, int PREC>
__global__ __launch_bounds__(BK * 2, 1) void bwd_dkdv_kernel(BwdParams p) {
  constexpr bool SPLIT = PREC == kPrecSplit;  // P and dS as hi + lo bf16 operand pairs
  constexpr int NW = BK / 32;
  static_assert(NW >= 2, "two waves copy lse2 and D");
  constexpr int TILE = BQ * D;                 // bf16 elements of one Q or dO tile
  constexpr int TB = TILE * 2;                 // its bytes
  // Q and dO tiles (three stages, swizzled; stage x holds Q then dO) and the
  // tile's lse2 / D rows.  Stage t % 3 holds tile t: tile t's scores are
  // computed while tile t - 1's dV/dK contributions (which read stage
  // (t-1) % 3) overlap the softmax-gradient math, and tile t + 1 is copied
  // into the third stage.
  __shared__ __attribute__((aligned(1024))) uint16_t sQO[3][2][TILE];
  __shared__ __attribute__((aligned(16))) float sL[3][BQ];
  __shared__ __attribute__((aligned(16))) float sD[3][BQ];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = int(uniform(uint32_t(tid >> 6)));  // wave-uniform by construction
  const int h = lane >> 5, lk = lane & 31;
  int kt, bh;
  xcd_coords(int(blockIdx.x), p.Tk_b, p.B * p.H, p.Tk_b < kInterleaveBelow, kt, bh);  // first key tiles are seen by the most rows
  const int head = bh % p.H, b = bh / p.H;
  const int N = p.N;
  const int k0 = kt * BK;
  const int key = k0 + wave * 32 + lk;
  const bool kvalid = key < N;
  const size_t base = size_t(b) * p.sb + size_t(head) * p.sh;
  const size_t rbase = (size_t(b) * p.H + head) * N;
  const __amdgpu_buffer_rsrc_t rQ = slice_rsrc(p.q + base, N, p.sn, D);
  const __amdgpu_buffer_rsrc_t rO = slice_rsrc(p.dO + base, N, p.sn, D);
  const __amdgpu_buffer_rsrc_t rL = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p.lse2 + rbase), 0, N * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rDv = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p.D + rbase), 0, N * 4, 0x00020000);
  TileDma<D, BQ, NW> dma;
  dma.init(wave, lane, p.sn);
  const uint32_t tile_bytes = uint32_t(BQ * p.sn * 2);
  auto issue = [&](int tile, int bf) {
    dma.issue(rQ, sQO[bf][0], uint32_t(tile) * tile_bytes);
    dma.issue(rO, sQO[bf][1], uint32_t(tile) * tile_bytes);
    if (wave == 0) dma_row_floats(rL, sL[bf], lane, uint32_t(tile * BQ * 4));
    else if (wave == 1) dma_row_floats(rDv, sD[bf], lane, uint32_t(tile * BQ * 4));
  };
  LdsOffsets<D, false> lo;
  lo.init(lane);

  // this wave's keys as B operands: K[key][16c + 8h ..], V[key][16c + 8h ..]
  bf16x8 kreg[D / 16], vreg[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    uint4 uk = make_uint4(0, 0, 0, 0), uv = make_uint4(0, 0, 0, 0);
    if (kvalid) {
      uk = *reinterpret_cast<const uint4*>(p.k + base + size_t(key) * p.sn + 16 * c + 8 * h);
      uv = *reinterpret_cast<const uint4*>(p.v + base + size_t(key) * p.sn + 16 * c + 8 * h);
    }
    kreg[c] = as_bf16x8(uk);
    vreg[c] = as_bf16x8(uv);
  }

  // this key column's visible query-row runs (in registers when at most MAXR)
  constexpr bool PRED = CHK == kCheckPredicate;
  const int nr = CAUSAL ? 1 : (PRED ? 0 : int(uniform(p.col_tkmax[size_t(b) * p.Tk_b + kt])));
  const uint2* myruns = (CAUSAL || PRED) ? nullptr : p.col_iv + (size_t(b) * N + (kvalid ? key : 0)) * p.K_c;
  PredSample ps;
  if constexpr (PRED) ps.init(p.pred, b, N);
  const LaneRuns<MAXR> runs =
      load_runs<MAXR>(CAUSAL, make_uint2(uint32_t(key), uint32_t(N)), myruns, nr, kvalid);

  f32x16 adv[D / 32], adk[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) { adv[db] = f32x16{}; adk[db] = f32x16{}; }

  TileIter it;
  int cnext = 0, clast = 0;
  if (!CAUSAL) it.init(p.bbm + (size_t(b) * p.Tk_b + kt) * p.Wb, p.Wb);
  else { cnext = k0 / BQ; clast = p.Tq_b - 1; }
  auto next_tile = [&](int& tile, int& state) -> bool {
    if (CAUSAL) {
      if (cnext > clast) return false;
      tile = cnext++;
      state = (tile * BQ >= k0 + BK - 1) ? 1 : 2;
      return true;
    }
    return it.next(tile, state);
  };

  int tile = 0, state = 0, buf = 0;
  bool have = next_tile(tile, state);
  if (have) issue(tile, 0);
  const char* lds0 = reinterpret_cast<const char*>(&sQO[0][0][0]);
  constexpr int NC = 4 * (D / 32);  // MFMAs of one of dV, dK per tile
  // dV^T += dO^T P (MFMAs 0..NC-1), dK^T += Q^T dS (NC..2NC-1) of the tile in
  // stage `st`; k = query, in the score-register order
  auto dvdk_read = [&](const char* st, int i) {
    const int j = i % NC, qc = j / (D / 32), dbk = j % (D / 32);
    const char* t = st + (i < NC ? TB : 0) + qc * (16 * D * 2);
    return lds_tr8_at(t + lo.tr(dbk, 0), t + lo.tr(dbk, 1));
  };
  // previous tile's P and dS (bf16; with the split precision also their low
  // parts); zero before the first tile
  constexpr int NL = SPLIT ? 4 : 1;
  bf16x8 ppb[4], pdb[4], ppl[NL], pdl[NL];
#pragma unroll
  for (int qc = 0; qc < 4; ++qc) {
    ppb[qc] = as_bf16x8(make_uint4(0, 0, 0, 0));
    pdb[qc] = as_bf16x8(make_uint4(0, 0, 0, 0));
  }
#pragma unroll
  for (int qc = 0; qc < NL; ++qc) {
    ppl[qc] = as_bf16x8(make_uint4(0, 0, 0, 0));
    pdl[qc] = as_bf16x8(make_uint4(0, 0, 0, 0));
  }
  int pbuf = 0;
  const bool any_tile = have;
  while (have) {
    const int ct = tile, cs = state;
    have = next_tile(tile, state);
    wait_vmem();
    __syncthreads();
    if (have) issue(tile, buf == 2 ? 0 : buf + 1);
    const char* cur = lds0 + buf * (2 * TB);
    const float* cL = sL[buf];
    const float* cD = sD[buf];

    // partial and ragged tiles: with the run bitmask the visibility is known
    // before the scores.  A tile none of this wave's key columns sees leaves
    // P = 0 without its S and dP MFMAs (its dS is then zero; the chunk phase
    // still carries the previous tile's dV/dK); one that all of them see
    // entirely runs unmasked.
    const bool masked = (cs == 2) || ((ct + 1) * BQ > N);
    WaveTile wt;
    wt.skip = false;
    wt.select = masked;
    if constexpr (CHK == kCheckRunBits) {
      if (masked) wt.init(tile_bits<MAXR>(uint32_t(ct * BQ + 4 * h), nr, runs, myruns, kvalid));
    }

    // S = Q K^T (NS MFMAs), then dP = dO V^T (NS MFMAs) in eight fenced
    // chunks, each also computing four probabilities P = exp2(S log2e/sqrt(d)
    // - lse2) of the finished S (lane = key column; its lse2 rows are read
    // one chunk ahead).
    f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
    if (!wt.skip) {
      constexpr int NS = D / 8, NM = 2 * NS, G = 4, MPC = NS / 8;
      auto rd = [&](int i) {
        const int j = i % NS;
        return lds_b128_at(cur + (i < NS ? 0 : TB) + (j & 1) * (32 * D * 2) + lo.row[j >> 1]);
      };
      auto mma = [&](int i, const bf16x8& a) {
        const int j = i % NS;
        if (i < NS) s[j & 1] = mfma32(a, kreg[j >> 1], s[j & 1]);
        else dp[j & 1] = mfma32(a, vreg[j >> 1], dp[j & 1]);
      };
      bf16x8 op[NM];
#pragma unroll
      for (int i = 0; i < G; ++i) op[i] = rd(i);
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        op[i + G] = rd(i + G);
        mma(i, op[i]);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, G, 0);
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      float4 l4n = *reinterpret_cast<const float4*>(cL + 4 * h);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int qb = c >> 2, vg = c & 3;
        const float4 l4 = l4n;
        if (c < 7) l4n = *reinterpret_cast<const float4*>(cL + ((c + 1) >> 2) * 32 + ((c + 1) & 3) * 8 + 4 * h);
#pragma unroll
        for (int m = 0; m < MPC; ++m) {
          const int i = NS + c * MPC + m;
          if (i + G < NM) op[i + G] = rd(i + G);
          mma(i, op[i]);
        }
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s[qb][vg * 4 + e] = __builtin_amdgcn_exp2f(fmaf(s[qb][vg * 4 + e], p.scale_log2, -lv[e]));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // invisible probabilities are zero
    if (wt.select && !wt.skip) {
      if constexpr (PRED) mask_pred<false>(s, uint32_t(ct * BQ + 4 * h), key, kvalid, ps, 0.f);
      else if constexpr (CHK == kCheckRunBits) apply_bits(s, wt.bits, 0.f);
      else mask_tile<CHK>(s, uint32_t(ct * BQ + 4 * h), nr, runs, myruns, kvalid, 0.f);
    }

    // dS = P (dP - D) of this tile and the bf16 P, dS operands, in eight
    // fenced chunks of four elements, each overlapped with 2NC/8 of the
    // previous tile's dV/dK MFMAs (operands read two MFMAs ahead, D one
    // chunk ahead).
    bf16x8 pb[4], db8[4], pl[NL], dl[NL];
    {
      constexpr int NM = 2 * NC, G = 2, MPC = NM / 8;
      const char* prv = lds0 + pbuf * (2 * TB);
      bf16x8 op[NM];
#pragma unroll
      for (int i = 0; i < G; ++i) op[i] = dvdk_read(prv, i);
      float4 d4n = *reinterpret_cast<const float4*>(cD + 4 * h);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int qb = c >> 2, vg = c & 3;
        const float4 d4 = d4n;
        if (c < 7) d4n = *reinterpret_cast<const float4*>(cD + ((c + 1) >> 2) * 32 + ((c + 1) & 3) * 8 + 4 * h);
#pragma unroll
        for (int m = 0; m < MPC; ++m) {
          const int i = c * MPC + m;
          if (i + G < NM) op[i + G] = dvdk_read(prv, i + G);
          const int j = i % NC, qc = j / (D / 32), dbk = j % (D / 32);
          if (i < NC) adv[dbk] = mfma32(op[i], ppb[qc], adv[dbk]);
          else adk[dbk] = mfma32(op[i], pdb[qc], adk[dbk]);
          if constexpr (SPLIT) {
            if (i < NC) adv[dbk] = mfma32(op[i], ppl[qc], adv[dbk]);
            else adk[dbk] = mfma32(op[i], pdl[qc], adk[dbk]);
          }
        }
        const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = vg * 4 + e;
          const float pe = s[qb][v];
          const float ds = pe * (dp[qb][v] - dv4[e]);
          const int qc = qb * 2 + (v >> 3), ee = v & 7;
          pb[qc][ee] = (__bf16)pe;
          db8[qc][ee] = (__bf16)ds;
          if constexpr (SPLIT) {
            pl[qc][ee] = bf16_lo(pe, pb[qc][ee]);
            dl[qc][ee] = bf16_lo(ds, db8[qc][ee]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int qc = 0; qc < 4; ++qc) { ppb[qc] = pb[qc]; pdb[qc] = db8[qc]; }
#pragma unroll
    for (int qc = 0; qc < NL; ++qc) { ppl[qc] = pl[qc]; pdl[qc] = dl[qc]; }
    pbuf = buf;
    buf = buf == 2 ? 0 : buf + 1;
  }
  // the last tile's dV/dK (its stage is still intact: no copy was issued after it)
  if (any_tile) {
    const char* prv = lds0 + pbuf * (2 * TB);
    mfma_stream<2 * NC, 4, 2, SPLIT ? 2 : 1>([&](int i) { return dvdk_read(prv, i); }, [&](int i, const bf16x8& a) {
      const int j = i % NC, qc = j / (D / 32), dbk = j % (D / 32);
      if (i < NC) adv[dbk] = mfma32(a, ppb[qc], adv[dbk]);
      else adk[dbk] = mfma32(a, pdb[qc], adk[dbk]);
      if constexpr (SPLIT) {
        if (i < NC) adv[dbk] = mfma32(a, ppl[qc], adv[dbk]);
        else adk[dbk] = mfma32(a, pdl[qc], adk[dbk]);
      }
    });
  }

  if (kvalid) {
    uint16_t* dKp = p.dk + base + size_t(key) * p.sn;
    uint16_t* dVp = p.dv + base + size_t(key) * p.sn;
#pragma unroll
    for (int dbk = 0; dbk < D / 32; ++dbk) {
#pragma unroll
      for (int vg = 0; vg < 4; ++vg) {
        bf16x4 k4, v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          k4[e] = (__bf16)(adk[dbk][vg * 4 + e] * p.scale);
          v4[e] = (__bf16)(adv[dbk][vg * 4 + e]);
        }
        *reinterpret_cast<bf16x4*>(dKp + dbk * 32 + vg * 8 + 4 * h) = k4;
        *reinterpret_cast<bf16x4*>(dVp + dbk * 32 + vg * 8 + 4 * h) = v4;
      }
    }
  }
}

// ------------------------------------------------------------------ dQ

template <int D, int BM, bool CAUSAL, int CHK, int PREC>
__global__ __launch_bounds__(BM * 2, BM == 128 ? 2 : 1) void bwd_dq_kernel(BwdParams p) {
  constexpr bool SPLIT = PREC == kPrecSplit;  // dS as hi + lo bf16 operand pairs
  constexpr int NW = BM / 32;
  constexpr int TILE = BN * D;
  constexpr int TB = TILE * 2;
  // K and V tiles in two stages (stage x holds K then V): tile t + 1 is
  // copied into the other stage while tile t is processed.  Two work-groups
  // share a CU, so one's vector math overlaps the other's matrix work.
  __shared__ __attribute__((aligned(1024))) uint16_t sKV[2][2][TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = int(uniform(uint32_t(tid >> 6)));  // wave-uniform by construction
  const int h = lane >> 5, lq = lane & 31;
  int kx, bh;
  xcd_coords(int(blockIdx.x), p.Tq_f, p.B * p.H, p.Tq_f < kInterleaveBelow, kx, bh);
  const int qt = p.Tq_f - 1 - kx;
  const int head = bh % p.H, b = bh / p.H;
  const int N = p.N;
  const int q0 = qt * BM;
  const int q = q0 + wave * 32 + lq;
  const bool qvalid = q < N;
  const size_t base = size_t(b) * p.sb + size_t(head) * p.sh;
  const size_t rbase = (size_t(b) * p.H + head) * N;
  const __amdgpu_buffer_rsrc_t rK = slice_rsrc(p.k + base, N, p.sn, D);
  const __amdgpu_buffer_rsrc_t rV = slice_rsrc(p.v + base, N, p.sn, D);
  TileDma<D, BN, NW> dma;
  dma.init(wave, lane, p.sn);
  const uint32_t tile_bytes = uint32_t(BN * p.sn * 2);
  LdsOffsets<D, true> lo;
  lo.init(lane);

  bf16x8 qreg[D / 16], oreg[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    uint4 uq = make_uint4(0, 0, 0, 0), uo = make_uint4(0, 0, 0, 0);
    if (qvalid) {
      uq = *reinterpret_cast<const uint4*>(p.q + base + size_t(q) * p.sn + 16 * c + 8 * h);
      uo = *reinterpret_cast<const uint4*>(p.dO + base + size_t(q) * p.sn + 16 * c + 8 * h);
    }
    qreg[c] = as_bf16x8(uq);
    oreg[c] = as_bf16x8(uo);
  }
  const float lse2 = qvalid ? p.lse2[rbase + q] : INFINITY;
  const float Dq = qvalid ? p.D[rbase + q] : 0.f;

  constexpr bool PRED = CHK == kCheckPredicate;
  const int nr = CAUSAL ? 1 : (PRED ? 0 : int(uniform(p.row_tkmax[size_t(b) * p.Tq_f + qt])));
  const uint2* myruns = (CAUSAL || PRED) ? nullptr : p.row_iv + (size_t(b) * N + (qvalid ? q : 0)) * p.K_r;
  PredSample ps;
  if constexpr (PRED) ps.init(p.pred, b, N);
  const LaneRuns<MAXR_Q> runs =
      load_runs<MAXR_Q>(CAUSAL, make_uint2(0u, uint32_t(q + 1)), myruns, nr, qvalid);

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

  TileIter it;
  int cnext = 0, clast = 0;
  if (!CAUSAL) it.init(p.fbm + (size_t(b) * p.Tq_f + qt) * p.Wf, p.Wf);
  else clast = min(p.Tk_f - 1, (q0 + BM - 1) / BN);
  auto next_tile = [&](int& tile, int& state) -> bool {
    if (CAUSAL) {
      if (cnext > clast) return false;
      tile = cnext++;
      state = ((tile + 1) * BN - 1 <= q0) ? 1 : 2;
      return true;
    }
    return it.next(tile, state);
  };

  int tile = 0, state = 0, buf = 0;
  bool have = next_tile(tile, state);
  if (have) {
    dma.issue(rK, sKV[0][0], uint32_t(tile) * tile_bytes);
    dma.issue(rV, sKV[0][1], uint32_t(tile) * tile_bytes);
  }
  const char* lds0 = reinterpret_cast<const char*>(&sKV[0][0][0]);
  constexpr int NQ = 4 * (D / 32);  // dQ MFMAs per tile
  while (have) {
    const int ct = tile, cs = state;
    have = next_tile(tile, state);
    wait_vmem();
    __syncthreads();  // every wave is done with the other stage
    if (have) {
      dma.issue(rK, sKV[buf ^ 1][0], uint32_t(tile) * tile_bytes);
      dma.issue(rV, sKV[buf ^ 1][1], uint32_t(tile) * tile_bytes);
    }
    const char* cur = lds0 + buf * (2 * TB);
    buf ^= 1;

    // partial and ragged tiles: with the run bitmask the visibility is known
    // before the scores; a tile none of this wave's rows sees is skipped, one
    // that all of them see entirely runs unmasked
    const bool masked = (cs == 2) || ((ct + 1) * BN > N);
    WaveTile wt;
    wt.skip = false;
    wt.select = masked;
    if constexpr (CHK == kCheckRunBits) {
      if (masked) wt.init(tile_bits<MAXR_Q>(uint32_t(ct * BN + 4 * h), nr, runs, myruns, qvalid));
    }
    if (wt.skip) continue;

    // S^T = K Q^T (NS MFMAs), then dP^T = V dO^T (NS MFMAs) in eight fenced
    // chunks, each also computing four probabilities of the finished S^T
    // (lane = query: one lse2 per lane).
    f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
    {
      constexpr int NS = D / 8, NM = 2 * NS, G = 2, MPC = NS / 8;
      auto rd = [&](int i) {
        const int j = i % NS;
        return lds_b128_at(cur + (i < NS ? 0 : TB) + (j & 1) * (32 * D * 2) + lo.row[j >> 1]);
      };
      auto mma = [&](int i, const bf16x8& a) {
        const int j = i % NS;
        if (i < NS) s[j & 1] = mfma32(a, qreg[j >> 1], s[j & 1]);
        else dp[j & 1] = mfma32(a, oreg[j >> 1], dp[j & 1]);
      };
      bf16x8 op[NM];
#pragma unroll
      for (int i = 0; i < G; ++i) op[i] = rd(i);
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        op[i + G] = rd(i + G);
        mma(i, op[i]);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, G, 0);
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int kb = c >> 2, vg = c & 3;
#pragma unroll
        for (int m = 0; m < MPC; ++m) {
          const int i = NS + c * MPC + m;
          if (i + G < NM) op[i + G] = rd(i + G);
          mma(i, op[i]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s[kb][vg * 4 + e] = __builtin_amdgcn_exp2f(fmaf(s[kb][vg * 4 + e], p.scale_log2, -lse2));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // invisible probabilities are zero
    if (wt.select) {
      if constexpr (PRED) mask_pred<true>(s, uint32_t(ct * BN + 4 * h), q, qvalid, ps, 0.f);
      else if constexpr (CHK == kCheckRunBits) apply_bits(s, wt.bits, 0.f);
      else mask_tile<CHK>(s, uint32_t(ct * BN + 4 * h), nr, runs, myruns, qvalid, 0.f);
    }

    // dQ^T += K^T dS^T: dS^T = P^T (dP^T - D) is packed to bf16 one 16-key
    // chunk at a time, fenced so that each chunk's MFMAs overlap the next
    // chunk's vector math (K read transposed, two MFMAs ahead).
    {
      constexpr int G = 2, MPK = D / 32;
      auto rd = [&](int i) {
        const int kc = i / (D / 32), db = i % (D / 32);
        const char* t = cur + kc * (16 * D * 2);
        return lds_tr8_at(t + lo.tr(db, 0), t + lo.tr(db, 1));
      };
      bf16x8 db8[4], dl8[SPLIT ? 4 : 1];
      bf16x8 op[NQ];
#pragma unroll
      for (int kc = 0; kc <= 4; ++kc) {
        if (kc == 0) {
#pragma unroll
          for (int i = 0; i < G; ++i) op[i] = rd(i);
        }
        if (kc > 0) {
#pragma unroll
          for (int m = 0; m < MPK; ++m) {
            const int i = (kc - 1) * MPK + m;
            if (i + G < NQ) op[i + G] = rd(i + G);
            acc[m] = mfma32(op[i], db8[kc - 1], acc[m]);
            if constexpr (SPLIT) acc[m] = mfma32(op[i], dl8[kc - 1], acc[m]);
          }
        }
        if (kc < 4) {
          const int kb = kc >> 1, v0 = (kc & 1) * 8;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float ds = s[kb][v0 + e] * (dp[kb][v0 + e] - Dq);
            db8[kc][e] = (__bf16)ds;
            if constexpr (SPLIT) dl8[kc][e] = bf16_lo(ds, db8[kc][e]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  if (qvalid) {
    uint16_t* dQp = p.dq + base + size_t(q) * p.sn;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int vg = 0; vg < 4; ++vg) {
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(acc[db][vg * 4 + e] * p.scale);
        *reinterpret_cast<bf16x4*>(dQp + db * 32 + vg * 8 + 4 * h) = o4;
      }
    }
  }
}

// Kernel choice for one (head dim, tile) pair: the check and the causal
// mode; the split precision exists for the default check only (the host
// refuses other combinations).  Both kernels take 2 * tile lanes.
struct DkdvLaunch {
  template <int D, int T, bool C, int CHK, int PREC>
  static void go(dim3 grid, const BwdParams& p, hipStream_t s) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, T, C, CHK, PREC>), grid, dim3(T * 2), 0, s, p);
  }
};
struct DqLaunch {
  template <int D, int T, bool C, int CHK, int PREC>
  static void go(dim3 grid, const BwdParams& p, hipStream_t s) {
    hipLaunchKernelGGL((bwd_dq_kernel<D, T, C, CHK, PREC>), grid, dim3(T * 2), 0, s, p);
  }
};

template <class L, int D, int T>
hipError_t dispatch(const AttnDims& a, dim3 grid, const BwdParams& p, hipStream_t s) {
  const bool c = a.causal != 0;
  if (a.precision == kPrecSplit) {
    if (c) L::template go<D, T, true, kCheckRunBits, kPrecSplit>(grid, p, s);
    else L::template go<D, T, false, kCheckRunBits, kPrecSplit>(grid, p, s);
  } else if (a.check == kCheckPredicate) {
    L::template go<D, T, false, kCheckPredicate, kPrecBf16>(grid, p, s);
  } else if (a.check == kCheckOrdinaryMasked) {
    if (c) L::template go<D, T, true, kCheckOrdinaryMasked, kPrecBf16>(grid, p, s);
    else L::template go<D, T, false, kCheckOrdinaryMasked, kPrecBf16>(grid, p, s);
  } else if (a.check == kCheckUnsigned) {
    if (c) L::template go<D, T, true, kCheckUnsigned, kPrecBf16>(grid, p, s);
    else L::template go<D, T, false, kCheckUnsigned, kPrecBf16>(grid, p, s);
  } else {
    if (c) L::template go<D, T, true, kCheckRunBits, kPrecBf16>(grid, p, s);
    else L::template go<D, T, false, kCheckRunBits, kPrecBf16>(grid, p, s);
  }
  return hipGetLastError();
}

BwdParams make_params(const AttnDims& a, const DescView& dv) {
  BwdParams p;
  std::memset(&p, 0, sizeof(p));
  p.sb = a.sb; p.sh = a.sh; p.sn = a.sn;
  p.B = a.B; p.H = a.H; p.N = a.N; p.d = a.d;
  p.scale = a.scale;
  p.scale_log2 = a.scale * kLog2e;
  p.Tq_f = (a.N + dv.fq - 1) / dv.fq;
  p.Tk_f = (a.N + dv.fk - 1) / dv.fk;
  p.Tk_b = (a.N + dv.bk - 1) / dv.bk;
  p.Tq_b = (a.N + dv.bq - 1) / dv.bq;
  p.Wf = dv.Wf; p.fbm = dv.fbm; p.row_iv = reinterpret_cast<const uint2*>(dv.row_iv); p.K_r = dv.K_r;
  p.row_tkmax = dv.row_tkmax;
  p.Wb = dv.Wb; p.bbm = dv.bbm; p.col_iv = reinterpret_cast<const uint2*>(dv.col_iv); p.K_c = dv.K_c;
  p.col_tkmax = dv.col_tkmax;
  p.pred.family = dv.pred.family; p.pred.tok_seg = dv.pred.tok_seg; p.pred.scalars = dv.pred.scalars;
  p.pred.n_scalars = dv.pred.n_scalars; p.pred.refs = dv.pred.refs; p.pred.seg_cap = dv.pred.seg_cap;
  p.pred.n_refs = dv.pred.n_refs; p.pred.sample_err = dv.pred.sample_err;
  return p;
}

}  // namespace

// ------------------------------------------------------------------ fixed scratch
//
// The backward's workspace (D and lse2 of every row) for callers that cannot
// allocate: a file-scope device array of kScratchRows rows, one copy per GPU,
// held until the process ends.  In host code `scratch` names a host-side
// stand-in; its device address comes from hipGetSymbolAddress, once per
// device with that device current, and only that address reaches kernels.
namespace {
static __device__ __align__(256) float scratch[2 * kScratchRows];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_workspace(float** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_bwd_dot(const AttnDims& a, const void* o, const void* dO, const float* lse, float* D,
                          hipStream_t stream) {
  DescView none;
  std::memset(&none, 0, sizeof(none));
  none.fq = none.fk = none.bk = none.bq = 64;
  BwdParams p = make_params(a, none);
  p.o = static_cast<const uint16_t*>(o);
  p.dO = static_cast<const uint16_t*>(dO);
  p.Dout = D;
  p.lse = lse;
  p.lse2out = D + size_t(a.B) * a.H * a.N;
  const int64_t rows = int64_t(a.B) * a.H * a.N;
  const int rpb = 256 / 4;  // four lanes per row
  dim3 grid(unsigned((rows + rpb - 1) / rpb));
  if (a.d == 128) hipLaunchKernelGGL(bwd_dot_kernel<128>, grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL(bwd_dot_kernel<64>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const AttnDims& a, const void* q, const void* k, const void* v, const float* lse,
                           const void* dO, const float* D, const DescView& dv, void* dk, void* dvv,
                           hipStream_t stream) {
  // 128-key tiles with the default check and bf16 operands: 64 keys per wave
  if (dkdv_wide_supported(a, dv)) return launch_bwd_dkdv_wide(a, q, k, v, dO, D, dv, dk, dvv, stream);
  BwdParams p = make_params(a, dv);
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.dO = static_cast<const uint16_t*>(dO);
  p.lse = lse;
  p.D = D;
  p.lse2 = D + size_t(a.B) * a.H * a.N;
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dvv);
  dim3 grid(p.Tk_b * a.H * a.B);
  if (a.d == 128) return dv.bk == 128 ? dispatch<DkdvLaunch, 128, 128>(a, grid, p, stream)
                                      : dispatch<DkdvLaunch, 128, 64>(a, grid, p, stream);
  return dv.bk == 128 ? dispatch<DkdvLaunch, 64, 128>(a, grid, p, stream) : dispatch<DkdvLaunch, 64, 64>(a, grid, p, stream);
}

hipError_t launch_bwd_dq(const AttnDims& a, const void* q, const void* k, const void* v, const float* lse,
                         const void* dO, const float* D, const DescView& dv, void* dq, hipStream_t stream) {
  BwdParams p = make_params(a, dv);
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.dO = static_cast<const uint16_t*>(dO);
  p.lse = lse;
  p.D = D;
  p.lse2 = D + size_t(a.B) * a.H * a.N;
  p.dq = static_cast<uint16_t*>(dq);
  dim3 grid(p.Tq_f * a.H * a.B);
  if (a.d == 128) return dv.fq == 128 ? dispatch<DqLaunch, 128, 128>(a, grid, p, stream)
                                      : dispatch<DqLaunch, 128, 64>(a, grid, p, stream);
  return dv.fq == 128 ? dispatch<DqLaunch, 64, 128>(a, grid, p, stream) : dispatch<DqLaunch, 64, 64>(a, grid, p, stream);
}

}  // namespace cm
