// attn_fwd.hip -- descriptor-guided attention forward (bf16 in, fp32 accumulate).
//
// CompileMask paper summary, section 3.3.2 "Descriptor-Guided Attention
// Execution": the Tile-State Bitmap lets the kernel skip empty tiles, run full
// tiles without a mask and check visibility only in partial tiles, with
// unsigned endpoint compares; invisible scores become -inf before the online
// softmax.  Section 2.1 "Background" describes the tiled kernel this extends.
//
// One work-group per (query tile of BM rows, head, sample); BM / 32 waves,
// each owning 32 query rows.  Scores are computed transposed, S^T = K Q^T, so
// a lane owns one query row: its visible runs sit in registers for the whole
// kernel, the partial-tile check is `(j - start) <u (end - start)` per run,
// and the row max / sum need one exchange with the lane holding the other 16
// keys of each 32-key block.  Key/value tiles of 64 rows are staged in LDS
// (row-major, padded); the next tile's global loads are in flight while the
// current one is computed.  O^T = V^T P^T reads V through transposed LDS
// reads and takes P^T straight from the score registers.
#include <hip/hip_runtime.h>

#include "attn_common.h"
#include "internal.h"

namespace cm {
namespace {

using namespace attn;

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int64_t sb, sh, sn;
  int32_t B, H, N;
  int32_t Tq, Tk;
  float scale_log2;
  const uint32_t* fbm;
  int32_t Wf;
  const uint2* row_iv;
  int32_t K_r;
  const uint32_t* row_tkmax;
  PredCtx pred;            // predicate baseline (check kCheckPredicate) only
};

constexpr int BN = 64;
constexpr int MAXR = 4;  // runs kept in registers; more are read from memory

template <int D, int BM, bool CAUSAL, int CHK, int PREC>
__global__ __launch_bounds__(BM * 2, BM == 128 ? 2 : 1) void attn_fwd_kernel(FwdParams p) {
  constexpr int NW = BM / 32;
  // K and V tiles, double-buffered, swizzled (see swz())
  __shared__ __attribute__((aligned(1024))) uint16_t sK[2][BN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sV[2][BN * D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = int(uniform(uint32_t(tid >> 6)));  // wave-uniform by construction
  const int h = lane >> 5, lq = lane & 31;
  int kx, bh;
  xcd_coords(int(blockIdx.x), p.Tq, p.B * p.H, p.Tq < kInterleaveBelow, kx, bh);
  const int qt = p.Tq - 1 - kx;  // the longest rows of lower-triangular masks first
  const int head = bh % p.H, b = bh / p.H;
  const int N = p.N;
  const int q0 = qt * BM;
  const int q = q0 + wave * 32 + lq;
  const bool qvalid = q < N;
  const size_t base = size_t(b) * p.sb + size_t(head) * p.sh;
  const __amdgpu_buffer_rsrc_t rK = slice_rsrc(p.k + base, N, p.sn, D);
  const __amdgpu_buffer_rsrc_t rV = slice_rsrc(p.v + base, N, p.sn, D);
  TileDma<D, BN, NW> dma;
  dma.init(wave, lane, p.sn);
  const uint32_t tile_bytes = uint32_t(BN * p.sn * 2);
  // per-lane byte offsets of the K row reads and V transposed reads; the
  // 32-key block and 16-key chunk offsets are immediates
  LdsOffsets<D, true> lo;
  lo.init(lane);

  // Q^T as MFMA B operands: lane holds Q[q][16c + 8h .. +7]
  bf16x8 qreg[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (qvalid) u = *reinterpret_cast<const uint4*>(p.q + base + size_t(q) * p.sn + 16 * c + 8 * h);
    qreg[c] = as_bf16x8(u);
  }

  // this row's visible runs (in registers when there are at most MAXR)
  constexpr bool PRED = CHK == kCheckPredicate;
  const int nr = CAUSAL ? 1 : (PRED ? 0 : int(uniform(p.row_tkmax[size_t(b) * p.Tq + qt])));
  const uint2* myruns = (CAUSAL || PRED) ? nullptr : p.row_iv + (size_t(b) * N + (qvalid ? q : 0)) * p.K_r;
  PredSample ps;
  if constexpr (PRED) ps.init(p.pred, b, N);
  const LaneRuns<MAXR> runs = load_runs<MAXR>(CAUSAL, make_uint2(0u, uint32_t(q + 1)), myruns, nr, qvalid);

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
  float m = -INFINITY, lsum = 0.f;

  // tile iteration
  TileIter it;
  int causal_next = 0, causal_last = 0;
  if (!CAUSAL) it.init(p.fbm + (size_t(b) * p.Tq + qt) * p.Wf, p.Wf);
  else causal_last = min(p.Tk - 1, (q0 + BM - 1) / BN);
  auto next_tile = [&](int& tile, int& state) -> bool {
    if (CAUSAL) {
      if (causal_next > causal_last) return false;
      tile = causal_next++;
      state = ((tile + 1) * BN - 1 <= q0) ? 1 : 2;
      return true;
    }
    return it.next(tile, state);
  };

  int tile = 0, state = 0, buf = 0;
  bool have = next_tile(tile, state);
  if (have) {
    dma.issue(rK, sK[0], uint32_t(tile) * tile_bytes);
    dma.issue(rV, sV[0], uint32_t(tile) * tile_bytes);
  }
  while (have) {
    const int ct = tile, cs = state;
    have = next_tile(tile, state);
    wait_vmem();       // this tile's copies have landed
    __syncthreads();   // ... for every wave; and nobody still reads the other buffer
    if (have) {
      dma.issue(rK, sK[buf ^ 1], uint32_t(tile) * tile_bytes);
      dma.issue(rV, sV[buf ^ 1], uint32_t(tile) * tile_bytes);
    }
    const char* cK = reinterpret_cast<const char*>(sK[buf]);
    const char* cV = reinterpret_cast<const char*>(sV[buf]);
    buf ^= 1;

    // partial tiles (and a ragged last tile): endpoint checks against the
    // row's runs.  With the run bitmask the visibility is known before the
    // scores: a tile that none of this wave's rows sees is skipped, and one
    // that all of them see entirely runs unmasked.
    const bool masked = (cs == 2) || ((ct + 1) * BN > N);
    WaveTile wt;
    wt.skip = false;
    wt.select = masked;
    if constexpr (CHK == kCheckRunBits) {
      if (masked) wt.init(tile_bits<MAXR>(uint32_t(ct * BN + 4 * h), nr, runs, myruns, qvalid));
    }
    if (wt.skip) continue;

    // S^T = K Q^T for two 32-key blocks (operand reads pipelined ahead).  The
    // wave raises its priority while it issues matrix instructions, so that
    // the SIMD's other wave does its softmax in the gaps rather than taking
    // issue slots from the matrix stream.
    f32x16 s[2] = {f32x16{}, f32x16{}};
    __builtin_amdgcn_s_setprio(2);
    mfma_stream<D / 8, 4, 1>(
        [&](int i) { return lds_b128_at(cK + (i & 1) * (32 * D * 2) + lo.row[i >> 1]); },
        [&](int i, const bf16x8& a) { s[i & 1] = mfma32(a, qreg[i >> 1], s[i & 1]); });
    __builtin_amdgcn_s_setprio(0);
    if (wt.select) {
      if constexpr (PRED) mask_pred<true>(s, uint32_t(ct * BN + 4 * h), q, qvalid, ps, -INFINITY);
      else if constexpr (CHK == kCheckRunBits) apply_bits(s, wt.bits, -INFINITY);
      else mask_tile<CHK>(s, uint32_t(ct * BN + 4 * h), nr, runs, myruns, qvalid, -INFINITY);
    }

    // online softmax in the log2 domain, scale folded into the exponent.  The
    // running max is only moved (and O rescaled) when some row's max grew by
    // more than 2^8; otherwise probabilities up to 256 are accumulated against
    // the stale max, which leaves O = acc / l unchanged.
    float mt = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mt = fmaxf(mt, s[kb][v]);
    mt = wave_xor32_max(mt) * p.scale_log2;
    if (__any(mt > m + 8.f)) {
      const float mn = fmaxf(m, mt);
      const float alpha = __builtin_amdgcn_exp2f(m - ((mn == -INFINITY) ? 0.f : mn));
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[db][v] *= alpha;
      m = mn;
    }
    const float mu = (m == -INFINITY) ? 0.f : m;
    float rsum = 0.f;
    constexpr bool SPLIT = PREC == kPrecSplit;
    bf16x8 pb[4], pl[SPLIT ? 4 : 1];
    // probabilities of elements [4 g, 4 g + 4) of key chunk kc (16 keys)
    auto probs = [&](int kc, int g) {
#pragma unroll
      for (int e = 4 * g; e < 4 * g + 4; ++e) {
        const float pe = __builtin_amdgcn_exp2f(fmaf(s[kc >> 1][(kc & 1) * 8 + e], p.scale_log2, -mu));
        rsum += pe;
        pb[kc][e] = (__bf16)pe;
        if constexpr (SPLIT) pl[kc][e] = bf16_lo(pe, pb[kc][e]);
      }
    };
    // key block 0 (chunks 0 and 1) now; key block 1 beside the PV MFMAs of
    // block 0, which do not need it
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      probs(kc, 0);
      probs(kc, 1);
    }

    // O^T += V^T P^T (V read transposed from LDS; with the split precision
    // each V operand multiplies P's high and low bf16 parts), in fenced steps
    // of one MFMA (two with the split precision); the operand reads run four
    // steps ahead, and steps 0, 2, 4, 6 of block 0 form a quarter of block 1's
    // probabilities each (pinned to their step)
    __builtin_amdgcn_s_setprio(2);
    {
      constexpr int NM = 4 * (D / 32), G = 4, NB0 = 2 * (D / 32);
      auto rd = [&](int i) {
        const int kc = i / (D / 32), db = i % (D / 32);
        const char* t = cV + kc * (16 * D * 2);
        return lds_tr8_at(t + lo.tr(db, 0), t + lo.tr(db, 1));
      };
      bf16x8 op[NM];
#pragma unroll
      for (int i = 0; i < G; ++i) op[i] = rd(i);
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        if (i + G < NM) op[i + G] = rd(i + G);
        acc[i % (D / 32)] = mfma32(op[i], pb[i / (D / 32)], acc[i % (D / 32)]);
        if constexpr (SPLIT) acc[i % (D / 32)] = mfma32(op[i], pl[i / (D / 32)], acc[i % (D / 32)]);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          if (i != x * NB0 / 4) continue;
          probs(2 + (x >> 1), x & 1);
          asm volatile("" : "+v"(pb[2 + (x >> 1)]), "+v"(rsum));
          if constexpr (SPLIT) asm volatile("" : "+v"(pl[2 + (x >> 1)]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    lsum += rsum;
    __builtin_amdgcn_s_setprio(0);
  }

  // epilogue: O = acc / l, lse = ln-sum-exp (natural log)
  const float lt = lsum + wave_xor32(lsum);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qvalid) {
    uint16_t* Op = p.o + base + size_t(q) * p.sn;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int vg = 0; vg < 4; ++vg) {
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(acc[db][vg * 4 + e] * inv);
        *reinterpret_cast<bf16x4*>(Op + db * 32 + vg * 8 + 4 * h) = o4;
      }
    }
    if (h == 0) {
      const float l2 = (m == -INFINITY || lt <= 0.f) ? -INFINITY : (m + __log2f(lt)) * kLn2;
      p.lse[(size_t(b) * p.H + head) * N + q] = l2;
    }
  }
}

template <int D, int BM, bool CAUSAL, int CHK, int PREC = kPrecBf16>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  dim3 grid(p.Tq * p.H * p.B);
  hipLaunchKernelGGL((attn_fwd_kernel<D, BM, CAUSAL, CHK, PREC>), grid, dim3(BM * 2), 0, stream, p);
  return hipGetLastError();
}

// (the split precision exists for the default check only: the host refuses
// other combinations)
template <int D, int BM>
hipError_t launch_dc(const FwdParams& p, bool causal, int check, int prec, hipStream_t stream) {
  if (prec == kPrecSplit)
    return causal ? launch<D, BM, true, kCheckRunBits, kPrecSplit>(p, stream)
                  : launch<D, BM, false, kCheckRunBits, kPrecSplit>(p, stream);
  if (check == kCheckPredicate) return launch<D, BM, false, kCheckPredicate>(p, stream);
  if (check == kCheckOrdinaryMasked)
    return causal ? launch<D, BM, true, kCheckOrdinaryMasked>(p, stream) : launch<D, BM, false, kCheckOrdinaryMasked>(p, stream);
  if (check == kCheckUnsigned)
    return causal ? launch<D, BM, true, kCheckUnsigned>(p, stream) : launch<D, BM, false, kCheckUnsigned>(p, stream);
  return causal ? launch<D, BM, true, kCheckRunBits>(p, stream) : launch<D, BM, false, kCheckRunBits>(p, stream);
}

}  // namespace

bool attn_tiles_supported(int d, int fq, int fk, int bk, int bq) {
  (void)d;
  return (fq == 64 || fq == 128) && fk == 64 && (bk == 64 || bk == 128) && bq == 64;
}

hipError_t launch_attn_fwd(const AttnDims& a, const void* q, const void* k, const void* v, const DescView& dv,
                           void* o, float* lse, hipStream_t stream) {
  FwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.sb = a.sb; p.sh = a.sh; p.sn = a.sn;
  p.B = a.B; p.H = a.H; p.N = a.N;
  p.Tq = (a.N + dv.fq - 1) / dv.fq;
  p.Tk = (a.N + dv.fk - 1) / dv.fk;
  p.scale_log2 = a.scale * attn::kLog2e;
  p.fbm = dv.fbm; p.Wf = dv.Wf; p.row_iv = reinterpret_cast<const uint2*>(dv.row_iv); p.K_r = dv.K_r;
  p.row_tkmax = dv.row_tkmax;
  p.pred.family = dv.pred.family; p.pred.tok_seg = dv.pred.tok_seg; p.pred.scalars = dv.pred.scalars;
  p.pred.n_scalars = dv.pred.n_scalars; p.pred.refs = dv.pred.refs; p.pred.seg_cap = dv.pred.seg_cap;
  p.pred.n_refs = dv.pred.n_refs; p.pred.sample_err = dv.pred.sample_err;
  const bool c = a.causal != 0;
  const int pr = a.precision;
  if (a.d == 128)
    return dv.fq == 128 ? launch_dc<128, 128>(p, c, a.check, pr, stream) : launch_dc<128, 64>(p, c, a.check, pr, stream);
  return dv.fq == 128 ? launch_dc<64, 128>(p, c, a.check, pr, stream) : launch_dc<64, 64>(p, c, a.check, pr, stream);
}

}  // namespace cm
