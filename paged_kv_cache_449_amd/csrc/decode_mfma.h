// Paged decode attention on the matrix cores, for query groups (several query
// heads per kv head).
//
// With G query heads per kv head, each K/V tile read through the block table
// serves G queries, so QK^T and PV are small dense contractions:
//   S[t][g] = sum_d K[t][d] q[g][d]          (16 tokens x G heads per tile)
//   O[g][d] += sum_t P[t][g] V[t][d]
// The tile is 16 tokens of one block (block_size >= 16) of one kv head.
//
//   QK  v_mfma_f32_16x16x32_{bf16,f16}: A = K rows (row i = token), B = q
//       (column j = head, zero for j >= G), D/32 steps over head_dim.  The K
//       tile is loaded contiguously and staged in LDS; lane (kg = lane/16,
//       t = lane%16) then reads the contiguous quarter [kg*D/4, (kg+1)*D/4)
//       of token t's row.  q is laid out with the same (kg, element) -> dim
//       mapping, so the contraction pairs matching dims whatever order the
//       instruction walks its k index in.
//   PV  v_mfma_f32_16x16x16_{bf16,f16}: A = V^T (row i = dim within a
//       16-column slice, k = token), B = P (k = token, column j = head).  The
//       QK result leaves lane (kg, j) holding S[4kg + r][j], r = 0..3, which
//       is exactly that lane's B operand (P[4kg + e][j]), so P never moves
//       between lanes.  V^T comes from the tile staged in LDS through the
//       gfx950 transposing read ds_read_b64_tr_b16: within each 16-lane
//       group, lane 4a + b receives element b of the 8-byte chunks that
//       lanes 4k + a (k = 0..3) address, so lane (kg, 4a + b) pointing its
//       own chunk at row 4kg + (lane%16)/4, columns 16dt + 4(lane%4) .. +3
//       receives V[4kg + k][16dt + 4a + b], k = 0..3: its A operand.
//
// fp8 pools are widened exactly to the operand type (E4M3FN is a subset of
// both bf16 and f16).  P enters PV as two operands of the operand type: its
// rounding and the rounding of the remainder (about 16 significant bits
// together); the running sum adds the fp32 weights.
// The online softmax keeps one running max per head (lanes j, j+16, j+32,
// j+48 agree on it) and per-lane partial sums that are added at the end.
#pragma once

namespace pkv {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// Operand type of the matrix instructions for a (KV, query) dtype pair; void
// where the pair runs on the vector ALUs instead.
template <typename KV, typename QT> struct mfma_operand { using type = void; };
template <> struct mfma_operand<bf16_t, bf16_t> { using type = bf16_t; };
template <> struct mfma_operand<f16_t, f16_t> { using type = f16_t; };
template <> struct mfma_operand<fp8_t, bf16_t> { using type = bf16_t; };
template <> struct mfma_operand<fp8_t, f16_t> { using type = f16_t; };

#define PKV_LDS __attribute__((address_space(3)))
typedef __bf16 lds_bf16x4 __attribute__((__vector_size__(8)));
typedef __fp16 lds_f16x4 __attribute__((__vector_size__(8)));

template <typename MT> struct mfma_ops;
template <> struct mfma_ops<bf16_t> {
  // transposing LDS read of four 16-bit values (see the file comment)
  __device__ static inline uint2 read_tr(const uint8_t* lds) {
    const PKV_LDS lds_bf16x4* p = (const PKV_LDS lds_bf16x4*)(lds);
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((PKV_LDS lds_bf16x4*)p));
  }
  // two fp8 codes (bytes 0,1 or 2,3 of w) -> two bf16, exact
  template <bool HI>
  __device__ static inline uint32_t from_fp8(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  }
  // two fp32 -> two bf16, round to nearest even
  __device__ static inline uint32_t pack(float a, float b) {
    bf16x2v v;
    v.x = (__bf16)a;
    v.y = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
  }
  __device__ static inline float lo(uint32_t w) { return __uint_as_float(w << 16); }
  __device__ static inline float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
  __device__ static inline f32x4 qk(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  }
  __device__ static inline f32x4 pv(uint2 a, uint2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                     0, 0, 0);
  }
};
template <> struct mfma_ops<f16_t> {
  __device__ static inline uint2 read_tr(const uint8_t* lds) {
    const PKV_LDS lds_f16x4* p = (const PKV_LDS lds_f16x4*)(lds);
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4f16((PKV_LDS lds_f16x4*)p));
  }
  template <bool HI>
  __device__ static inline uint32_t from_fp8(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
  }
  __device__ static inline uint32_t pack(float a, float b) {
    half2v v;
    v.x = (_Float16)a;
    v.y = (_Float16)b;
    return __builtin_bit_cast(uint32_t, v);
  }
  __device__ static inline float lo(uint32_t w) { return (float)__builtin_bit_cast(half2v, w).x; }
  __device__ static inline float hi(uint32_t w) { return (float)__builtin_bit_cast(half2v, w).y; }
  __device__ static inline f32x4 qk(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  }
  __device__ static inline f32x4 pv(uint2 a, uint2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0,
                                                 0, 0);
  }
};

// Operand type of PV.  fp8 codes and f16 values are exact in f16, and
// the weights P rounded once to f16 (relative error 2^-11) move an output by
// at most 2^-11 of the largest |v| it averages, far inside the tolerance:
// those pools take one f16 P operand.  bf16 values are not exact in f16 (its
// range is smaller), and P rounded to bf16 (2^-8) is not accurate enough,
// so bf16 pools take P as a rounded bf16 head plus the rounded remainder
// (two PV instructions).
template <typename KV, typename MT>
struct pv_operand {
  using type = typename std::conditional<std::is_same<MT, bf16_t>::value && elem_size<KV>::value == 2, bf16_t,
                                         f16_t>::type;
  static constexpr bool split = std::is_same<type, bf16_t>::value;
};

template <typename KV, int D>
struct MfmaShape {
  static constexpr int EB = elem_size<KV>::value;
  static constexpr int ROW = D * EB;             // bytes of one token row
  static constexpr int KL = ROW / 64;            // 16-byte loads per lane: a quarter row
  static constexpr int VL = 16 * ROW / 1024;     // wave loads of one 16-token V tile
  static constexpr int KS = D / 32;              // QK instructions per tile
  static constexpr int DT = D / 16;              // PV instructions per tile (16 dims each)
  // LDS bytes per staged V row (operand type): 32 bytes past a multiple of
  // 256 for D = 128 and 256, so the 16 rows x 32 bytes a transposing read
  // touches spread over all banks
  static constexpr int LSTRIDE = 2 * D + 32;
  // K tiles are loaded contiguously and staged in LDS: a lane reading its own
  // token's quarter row straight from memory makes each load touch 16 lines,
  // which stalled the address units on the L1 (for about a third of the
  // kernel on 128-byte fp8 rows).  Rows are padded by 16 bytes so the 16 rows
  // of a read fall in different banks.
  static constexpr int KSTRIDE = ROW + 16;
  static_assert(KL >= 1 && VL >= 1 && KS >= 1 && KL == VL, "tile shape");
};

template <typename KV, int D>
struct MfmaTileRegs {
  uint4 k[MfmaShape<KV, D>::KL];
  uint4 v[MfmaShape<KV, D>::VL];
};

// Tiles loaded and computed together in one pipeline step.  Two tiles per
// step (PV paired into 16x16x32 steps, 8 KiB of fp8 in flight per wave)
// measured 11% slower than one on the fp8 GQA decode workload on MI355X,
// so runs take one tile per step; the paired form stays for TPS = 2.
template <typename KV, int D>
struct MfmaStep {
  static constexpr int TPS = 1;
  MfmaTileRegs<KV, D> t[TPS];
};

// LDS staging of a matrix-core run's tiles (V as the operand type, K as
// loaded).  One pair of arrays per (dtype, head dim), shared by every run of
// a kernel whatever its cache policy: the runs of a one-wave work-group
// follow one another.
template <typename KV, int D>
struct MfmaStage {
  __device__ static uint8_t* v() {
    __shared__ __attribute__((aligned(16))) uint8_t a[MfmaStep<KV, D>::TPS * 16 * MfmaShape<KV, D>::LSTRIDE];
    return a;
  }
  __device__ static uint8_t* k() {
    __shared__ __attribute__((aligned(16))) uint8_t a[MfmaStep<KV, D>::TPS * 16 * MfmaShape<KV, D>::KSTRIDE];
    return a;
  }
};

// Lazy rescaling: a run's reference max moves only when a row's max passes
// it by more than this (log2 units), so weights stay below 2^8 and the
// accumulator is rescaled rarely rather than at every tile.
constexpr float kRescaleSlack = 8.0f;

// Issue the loads of 16-token tile j of the current table window (tokens
// tlo + 16j ...).  Tokens at or past thi and blocks whose table entry is out
// of range read as zeros.
template <typename KV, int D, int POL>
__device__ inline void mfma_issue(const RunCtx& c, int tab, int tlo, int thi, int j, MfmaTileRegs<KV, D>& r) {
  using Sh = MfmaShape<KV, D>;
  const int lane = threadIdx.x & 63;
  // the tile index and window are wave-uniform (the work-group kernels derive
  // j from the wave index): say so, so the descriptors stay scalar
  j = __builtin_amdgcn_readfirstlane(j);
  tlo = __builtin_amdgcn_readfirstlane(tlo);
  thi = __builtin_amdgcn_readfirstlane(thi);
  const int bi = min((j * 16) >> c.log2_bs, 63);
  const int phys = __builtin_amdgcn_readlane(tab, bi);
  const int t0 = tlo + j * 16;             // first token of the tile
  const int o0 = (j * 16) & c.bs_mask;     // its slot in the block (tiles never straddle blocks)
  // The descriptors start at the tile and cover only its rows inside the
  // window: rows at or past thi, and every row of a block whose table entry
  // is out of range (-1), fall outside them and read as zeros, with no
  // per-lane compare.  The lane offsets are then the same for every tile.
  const int rows = __builtin_amdgcn_readfirstlane(phys < 0 ? 0 : max(0, min(16, thi - t0)));
  const int64_t toff = c.blk_stride * max(phys, 0) + (int64_t)o0 * Sh::ROW;
  const uint32_t nrec = (uint32_t)(rows * Sh::ROW);
  __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)(c.k_head + toff), (short)0, (int)nrec, kBufferWord3);
  __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void*)(c.v_head + toff), (short)0, (int)nrec, kBufferWord3);
  // K and V: the 16 x ROW tiles, contiguous, 16 bytes per lane per wave load
#pragma unroll
  for (int q = 0; q < Sh::KL; ++q)
    r.k[q] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, (q * 64 + lane) * 16, 0, POL));
#pragma unroll
  for (int u = 0; u < Sh::VL; ++u)
    r.v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, (u * 64 + lane) * 16, 0, POL));
}

// K operand words of QK step st (8 elements of the operand type) from the
// lane's quarter row.
template <typename KV, typename MT, int D>
__device__ inline uint4 mfma_k_operand(const uint4 (&kq)[MfmaShape<KV, D>::KL], int st) {
  if constexpr (elem_size<KV>::value == 2) {
    return kq[st];
  } else {
    // fp8: step st uses bytes 8st .. 8st+7 of the quarter row
    const uint4 w = kq[st >> 1];
    const uint32_t a = (st & 1) ? w.z : w.x;
    const uint32_t b = (st & 1) ? w.w : w.y;
    return make_uint4(mfma_ops<MT>::template from_fp8<false>(a), mfma_ops<MT>::template from_fp8<true>(a),
                      mfma_ops<MT>::template from_fp8<false>(b), mfma_ops<MT>::template from_fp8<true>(b));
  }
}

// Cuts inside a run: a run that crosses chunk boundaries leaves the state
// of each finished chunk's part as that chunk's record and starts the next
// part from zero, without leaving its load pipeline.  `first` and `every`
// count 16-token tiles: to the first cut, and between cuts; `cuts` is their
// number (a run that ends on a chunk boundary has no cut there: its last
// part is the caller's); the functor stores part k.  NoCut: one part.
struct NoCut {
  static constexpr bool kActive = false;
  int first = 0, every = 0, cuts = 0;
  template <int DT>
  __device__ void operator()(int, const f32x4 (&)[DT], float, float) const {}
};

// Query row served by lane (kg, j) of a matrix-core run.
struct MfmaRow {
  bool valid;     // row j holds a query
  int64_t qoff;   // element offset of its q row (and of its out row)
  int limit;      // tokens at or past this index are masked for the row
  int min_limit;  // the smallest limit of the run's valid rows (uniform)
  int64_t part;   // PART runs: index of the row's partial record
};

// max of n values (n >= 3), folded two at a time into a running max so each
// step is one v_maximum3_f32 (NaN propagates)
template <int N>
__device__ inline float max_of(const float* v) {
  static_assert(N >= 3, "three or more values");
  float m = __builtin_elementwise_maximum(__builtin_elementwise_maximum(v[0], v[1]), v[2]);
#pragma unroll
  for (int i = 3; i + 1 < N; i += 2) m = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m, v[i]), v[i + 1]);
  if constexpr (N % 2 == 0) m = __builtin_elementwise_maximum(m, v[N - 1]);
  return m;
}

// max of x over lanes l, l ^ 16, l ^ 32 and l ^ 48: the 32-lane halves,
// then the 16-lane rows, swapped between two copies of x (VALU, no LDS).
__device__ inline float lane_max_xor32_xor16(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// One run of up to 16 query rows against blocks [off, off+len) of the
// (kv head h, sequence s) stream, which has nb blocks and n tokens; `rows`
// maps record row j to the element offset of its out row (-1: no query).
// R is the number of record rows.  All scalars are uniform.
//
// PART runs (whole runs only) leave each valid row's unnormalised state
// (acc[D], reference max, sum) as record row.part of p.partials instead of
// writing out, for a later kernel to continue.
//
// mfma_rows_core runs the stream and leaves the run's state: lane (kg, j16)
// holds acc[dt] = O[j16][16 dt + 4kg + i], i = 0..3 (unnormalised), the
// row's reference max m (log2 units) and its whole running sum l.
template <typename KV, typename QT, int D, int POL, typename Cut = NoCut>
__device__ inline void mfma_rows_core(const DecodeParams& p, int s, int h, int off, int len, int n,
                                      const MfmaRow& row, f32x4 (&acc)[MfmaShape<KV, D>::DT], float& m, float& l,
                                      const Cut& cut = Cut{}) {
  using MT = typename mfma_operand<KV, QT>::type;
  using Ops = mfma_ops<MT>;
  using PT = typename pv_operand<KV, MT>::type;
  using PVOps = mfma_ops<PT>;
  constexpr bool kSplitP = pv_operand<KV, MT>::split;
  using Sh = MfmaShape<KV, D>;
  constexpr int KS = Sh::KS, DT = Sh::DT, LSTRIDE = Sh::LSTRIDE;
  constexpr int TPS = MfmaStep<KV, D>::TPS;
  constexpr int QE = elem_size<QT>::value;
  uint8_t* vlds = MfmaStage<KV, D>::v();
  uint8_t* klds = MfmaStage<KV, D>::k();

  const int lane = threadIdx.x;
  const int j16 = lane & 15;   // token row (QK A) / query row (B, D)
  const int kg = lane >> 4;    // k group
  // Scores are scaled inside the exponent, exp2(sc * qabs - mu), and their
  // max is taken before scaling, which needs a positive scale: a negative
  // one flips the sign of the q operand instead (exact).  A zero scale
  // becomes 1e-30, under which every score still rounds to exp2(0) = 1 and
  // masked ones stay -inf.
  const float qsc = run_q_scale(p, h);
  const float qabs = fmaxf(fabsf(qsc), 1e-30f);
  const uint32_t qflip = qsc < 0.0f ? 0x80008000u : 0u;

  // q operand: lane (kg, j) holds q row j at dims kg*D/4 + 8st .. +8 for step st
  uint4 qop[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st) qop[st] = make_uint4(0u, 0u, 0u, 0u);
  if (row.valid) {
    const int64_t qe = row.qoff + kg * (D / 4);
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      const uint4 w4 = *(const uint4*)(p.q + (qe + st * 8) * QE);
      qop[st] = make_uint4(w4.x ^ qflip, w4.y ^ qflip, w4.z ^ qflip, w4.w ^ qflip);
    }
  }

#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  m = -INFINITY;   // reference max of row j16 (log2 units)
  l = 0.0f;        // this lane's share of the running sum, until the end
  float mu = 0.0f; // m as the exponent offset (0 while m is -inf)

  RunCtx c;
  const int64_t tile = (int64_t)Sh::ROW << p.log2_bs;
  c.k_head = p.k_pool + tile * h;
  c.v_head = p.v_pool + tile * h;
  c.blk_stride = tile * p.num_kv_heads;
  c.tile_bytes = (uint32_t)tile;
  c.lane_off = 0;
  c.row_bytes = Sh::ROW;
  c.log2_bs = p.log2_bs;
  c.bs_mask = (1 << p.log2_bs) - 1;
  const int32_t* trow = p.block_tables + (int64_t)s * p.max_blocks + off;
  static_assert(!Cut::kActive || TPS == 1, "cuts fall between single-tile steps");
  int to_cut = cut.first, part = 0;

  // One pipeline step: TPS tiles staged in LDS (V as the operand type, rows
  // padded to LSTRIDE; K as loaded, rows padded to KSTRIDE), QK for each, one
  // online-softmax update for the step, then PV.  With two tiles, PV runs
  // 16x16x32 steps whose contraction index 8kg + e stands for token 4kg + e
  // of the first tile (e < 4) and 4kg + e - 4 of the second, on both
  // operands.
  auto compute = [&](const MfmaStep<KV, D>& r, int tab, int tlo, int thi, int st, int unmasked_end, bool real) {
    __syncthreads();   // the previous step's LDS reads are done
#pragma unroll
    for (int q = 0; q < TPS; ++q) {
#pragma unroll
      for (int u = 0; u < Sh::VL; ++u) {
        const int byte = (u * 64 + lane) * 16;
        const int vr = byte / Sh::ROW, ve = (byte % Sh::ROW) / Sh::EB;   // row, first element
        uint8_t* dst = vlds + (q * 16 + vr) * LSTRIDE + ve * 2;
        if constexpr (Sh::EB == 2) {
          *(uint4*)dst = r.t[q].v[u];
        } else {
          const uint4 w4 = r.t[q].v[u];
          *(uint4*)dst = make_uint4(PVOps::template from_fp8<false>(w4.x), PVOps::template from_fp8<true>(w4.x),
                                    PVOps::template from_fp8<false>(w4.y), PVOps::template from_fp8<true>(w4.y));
          *(uint4*)(dst + 16) = make_uint4(PVOps::template from_fp8<false>(w4.z), PVOps::template from_fp8<true>(w4.z),
                                           PVOps::template from_fp8<false>(w4.w), PVOps::template from_fp8<true>(w4.w));
        }
        *(uint4*)(klds + (q * 16 + vr) * Sh::KSTRIDE + (byte % Sh::ROW)) = r.t[q].k[u];
      }
    }
    __syncthreads();
    // S^T tiles: lane (kg, j16) gets scores of tokens 4kg + i, i = 0..3, row j16
    f32x4 sc[TPS];
#pragma unroll
    for (int q = 0; q < TPS; ++q) {
      uint4 kq[Sh::KL];
#pragma unroll
      for (int w = 0; w < Sh::KL; ++w)
        kq[w] = *(const uint4*)(klds + (q * 16 + j16) * Sh::KSTRIDE + kg * (Sh::ROW / 4) + w * 16);
      sc[q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < KS; ++k) sc[q] = Ops::qk(mfma_k_operand<KV, MT, D>(kq, k), qop[k], sc[q]);
    }
    float x[TPS][4];
#pragma unroll
    for (int q = 0; q < TPS; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[q][i] = sc[q][i];   // raw: qabs * score is in log2 units
    if (tlo + (st + 1) * TPS * 16 > unmasked_end) {   // some token of the step may be masked
      const int lim = min(thi, row.limit);
#pragma unroll
      for (int q = 0; q < TPS; ++q) {
        const int j = st * TPS + q;
        const bool bvalid = __builtin_amdgcn_readlane(tab, min((j * 16) >> p.log2_bs, 63)) >= 0;
        const int t0 = tlo + j * 16 + 4 * kg;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!(bvalid && t0 + i < lim)) x[q][i] = -INFINITY;
      }
    }
    // the row's max: the lane's values, then the four lane groups kg of the
    // row by two half swaps (NaN propagates, as through the exponentials)
    const float mx = lane_max_xor32_xor16(max_of<TPS * 4>(&x[0][0])) * qabs;
    if (__ballot(mx > m + kRescaleSlack)) {
      const float mn = fmaxf(m, mx);
      const float alpha = m == -INFINITY ? 0.0f : fexp2(m - mn);
      m = mn;
      mu = mn == -INFINITY ? 0.0f : mn;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
    }
    // weights: one f16 operand where V is exact in f16 (fp8 codes, f16),
    // else (bf16) a rounded head plus the rounded remainder -- one bf16
    // operand alone (8 significant bits) would leave an error of up to ~2^-8
    // of the spread of V in rows that see few tokens, f16's 2^-11 stays well
    // inside the tolerance
    uint32_t ph[TPS][2], pr[TPS][2];
#pragma unroll
    for (int q = 0; q < TPS; ++q) {
      float e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) e[i] = fexp2(__builtin_fmaf(x[q][i], qabs, -mu));
      l += (e[0] + e[1]) + (e[2] + e[3]);
      ph[q][0] = PVOps::pack(e[0], e[1]);
      ph[q][1] = PVOps::pack(e[2], e[3]);
      if constexpr (kSplitP) {
        pr[q][0] = PVOps::pack(e[0] - PVOps::lo(ph[q][0]), e[1] - PVOps::hi(ph[q][0]));
        pr[q][1] = PVOps::pack(e[2] - PVOps::lo(ph[q][1]), e[3] - PVOps::hi(ph[q][1]));
      }
    }
    // lane (kg, i) needs V[4kg + e][16 dt + i], e = 0..3: one transposing read per tile
    const uint8_t* tr = vlds + (4 * kg + (j16 >> 2)) * LSTRIDE + (lane & 3) * 8;
    if constexpr (TPS == 2) {
      const uint4 bh = make_uint4(ph[0][0], ph[0][1], ph[1][0], ph[1][1]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint2 va = PVOps::read_tr(tr + dt * 32);
        const uint2 vb = PVOps::read_tr(tr + 16 * LSTRIDE + dt * 32);
        const uint4 a = make_uint4(va.x, va.y, vb.x, vb.y);
        acc[dt] = PVOps::qk(a, bh, acc[dt]);
        if constexpr (kSplitP) acc[dt] = PVOps::qk(a, make_uint4(pr[0][0], pr[0][1], pr[1][0], pr[1][1]), acc[dt]);
      }
    } else {
      const uint2 bh = make_uint2(ph[0][0], ph[0][1]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const auto vt = PVOps::read_tr(tr + dt * 32);
        acc[dt] = PVOps::pv(vt, bh, acc[dt]);
        if constexpr (kSplitP) acc[dt] = PVOps::pv(vt, make_uint2(pr[0][0], pr[0][1]), acc[dt]);
      }
    }
    if constexpr (Cut::kActive) {
      // the tile ends a chunk: its part is done (a step past the window,
      // issued only to keep the wait counts exact, is no tile)
      if (real && part < cut.cuts && --to_cut == 0) {
        float lt = l;
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        cut(part, acc, m, lt);
        ++part;
        to_cut = cut.every;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        m = -INFINITY;
        l = 0.0f;
        mu = 0.0f;
      }
    }
  };

  int tab = load_table_window(p, trow, 0, len);
  for (int wb = 0; wb < len; wb += 64) {
    const int cnt = min(64, len - wb);
    const int tab_next = wb + 64 < len ? load_table_window(p, trow, wb + 64, len) : -1;
    const int tlo = (off + wb) << p.log2_bs;
    const int thi = min((off + wb + cnt) << p.log2_bs, n);
    const int tiles = (thi - tlo + 15) >> 4;
    // tokens below this need no mask: every row of the run sees them and
    // every table entry of the window is in the pool
    const bool all_in_pool = __ballot(lane < cnt && tab < 0) == 0;
    const int unmasked_end = all_in_pool ? min(thi, row.min_limit) : tlo;
    // fp8 keeps two step register sets in flight (issue the next step,
    // compute this one); 16-bit elements issue and compute one set, whose
    // loads already carry twice the bytes.  On MI355X two sets were 10-12%
    // faster for fp8 GQA decode with the library-sized split (3% slower
    // with 512-token partitions), and one set 2-5% faster for bf16 and f16
    // (GQA decode, grouped decode, speculative verification).  Issues are
    // unconditional so the compiler's wait counts stay exact (a tile past
    // the window reads zeros and its scores are all masked).
    const int steps = (tiles + TPS - 1) / TPS;
    MfmaStep<KV, D> a;
    auto issue = [&](MfmaStep<KV, D>& r, int st) {
#pragma unroll
      for (int q = 0; q < TPS; ++q) mfma_issue<KV, D, POL>(c, tab, tlo, thi, st * TPS + q, r.t[q]);
    };
    if constexpr (Sh::EB == 1) {
      MfmaStep<KV, D> b;
      issue(a, 0);
      for (int st = 0; st < steps; st += 2) {
        issue(b, st + 1);
        compute(a, tab, tlo, thi, st, unmasked_end, true);
        issue(a, st + 2);
        compute(b, tab, tlo, thi, st + 1, unmasked_end, st + 1 < steps);
      }
    } else {
      for (int st = 0; st < steps; ++st) {
        issue(a, st);
        compute(a, tab, tlo, thi, st, unmasked_end, true);
      }
    }
    tab = tab_next;
  }

  // total sum of row j16 over the four k groups
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
}

// Matrix-core state of a part -> its record (rows j16 < R of valid lanes).
template <typename KV, int D>
__device__ inline void mfma_store_record(const RecordRef& rec, bool valid, const f32x4 (&acc)[MfmaShape<KV, D>::DT],
                                         float m, float l) {
  constexpr int DT = MfmaShape<KV, D>::DT;
  const int j16 = threadIdx.x & 15, kg = threadIdx.x >> 4;
  if (valid) {
    const int rg = j16 * (D + 4);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      record_store4(rec, rg + dt * 16 + 4 * kg, acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
    if (kg == 0) record_store4(rec, rg + D, m, l, 0.0f, 0.0f);
  }
}

// The parts a run leaves in the chunks it crosses: part k goes to chunk
// v0 + k, as the chunk's first part (slot 0), except part 0 of a run that
// starts inside its chunk (slot 1).
//
// The first NP parts wait in LDS until the run ends.  A record stored in the
// middle of the stream would hold up the run: a wave's vector memory
// operations complete in issue order, so the next tile's loads would wait
// for the stores to be written through.  NP fits the LDS a work-group may
// hold with 8 per CU (20 KiB, the tile staging included); parts past NP are
// stored at once.
template <typename KV, int D, int R>
struct RecordCuts {
  static constexpr bool kActive = true;
  static constexpr int kRec = R * (D + 4);   // floats per part
  static constexpr int kStage =
      MfmaStep<KV, D>::TPS * 16 * (MfmaShape<KV, D>::LSTRIDE + MfmaShape<KV, D>::KSTRIDE);
  static constexpr int kFit = kStage + kRec * 4 > 20480 ? 0 : (20480 - kStage) / (kRec * 4);
  static constexpr int NP = kFit > 8 ? 8 : kFit;
  int first, every, cuts;
  float* partials;
  int v0, slot0;
  bool valid;
  __device__ static float* lds() {
    __shared__ __attribute__((aligned(16))) float a[NP > 0 ? NP * kRec : 4];
    return a;
  }
  __device__ RecordRef record(int k) const {
    return record_ref<D, R>(partials + (int64_t)(2 * (v0 + k) + (k == 0 ? slot0 : 0)) * kRec);
  }
  __device__ void operator()(int k, const f32x4 (&acc)[MfmaShape<KV, D>::DT], float m, float l) const {
    constexpr int DT = MfmaShape<KV, D>::DT;
    if (k < NP) {   // the lane's own elements, as it will store them
      const int j16 = threadIdx.x & 15, kg = threadIdx.x >> 4;
      float* b = lds() + k * kRec + j16 * (D + 4);
      if (valid) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) *(f32x4*)(b + dt * 16 + 4 * kg) = acc[dt];
        if (kg == 0) *(float2*)(b + D) = make_float2(m, l);
      }
    } else {
      mfma_store_record<KV, D>(record(k), valid, acc, m, l);
    }
  }
  // store the parts held in LDS (each lane reads back what it wrote)
  __device__ void flush() const {
    constexpr int DT = MfmaShape<KV, D>::DT;
    const int j16 = threadIdx.x & 15, kg = threadIdx.x >> 4;
    for (int k = 0; k < min(cuts, NP); ++k) {
      const float* b = lds() + k * kRec + j16 * (D + 4);
      const RecordRef rec = record(k);
      if (valid) {
        const int rg = j16 * (D + 4);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const f32x4 x = *(const f32x4*)(b + dt * 16 + 4 * kg);
          record_store4(rec, rg + dt * 16 + 4 * kg, x[0], x[1], x[2], x[3]);
        }
        if (kg == 0) {
          const float2 ml = *(const float2*)(b + D);
          record_store4(rec, rg + D, ml.x, ml.y, 0.0f, 0.0f);
        }
      }
    }
  }
};

// CUTS: the run may cross chunk boundaries of the grid (a worker streaming a
// span of partitions), leaving one record per chunk crossed.
template <typename KV, typename QT, int D, int R, int POL, typename Rows, bool PART = false, bool CUTS = false>
__device__ inline void mfma_rows_run(const DecodeParams& p, int w, const ChunkGrid& grid, int wstart, int pos, int s,
                                     int h, int off, int len, int n, int nb, const MfmaRow& row, const Rows& rows) {
  using Sh = MfmaShape<KV, D>;
  static_assert(R >= 1 && R <= 16, "query rows");
  constexpr int DT = Sh::DT;
  constexpr int QE = elem_size<QT>::value;
  const int lane = threadIdx.x;
  const int j16 = lane & 15;
  const int kg = lane >> 4;
  // the chunks the whole run spans (worked out before the run, while few
  // registers are live)
  const int seg_start = pos - off;
  const int first_w = grid.of(seg_start);
  const int last_w = grid.of(seg_start + nb - 1);
  f32x4 acc[DT];
  float m, l;
  int pieces = 1;    // records this run leaves
  int last_v = w;    // chunk of its last part
  if constexpr (CUTS) {
    last_v = grid.of(pos + len - 1);
    pieces = last_v - w + 1;
  }
  if (CUTS && pieces > 1) {
    // cuts fall on chunk starts, every grid.chunk blocks within the span
    const int tpb = 1 << (p.log2_bs - 4);   // tiles per block
    const RecordCuts<KV, D, R> cut{(grid.start(w + 1) - pos) * tpb, grid.chunk * tpb, pieces - 1, p.partials, w,
                                   pos == wstart ? 0 : 1, row.valid && j16 < R};
    mfma_rows_core<KV, QT, D, POL>(p, s, h, off, len, n, row, acc, m, l, cut);
    cut.flush();
  } else {
    mfma_rows_core<KV, QT, D, POL>(p, s, h, off, len, n, row, acc, m, l);
  }
  const float vs = run_v_scale(p, h);

  // lane (kg, j16) holds O[j16][16 dt + 4kg + i], i = 0..3
  if constexpr (PART) {
    if (row.valid) {
      float* rec = p.partials + row.part * (D + 4);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) *(f32x4*)(rec + dt * 16 + 4 * kg) = acc[dt];
      if (kg == 0) *(float2*)(rec + D) = make_float2(m, l);
    }
    return;
  }
  if (off == 0 && off + len == nb && pieces == 1) {   // the whole run is ours
    if (row.valid) {
      const float mul = l > 0.0f ? vs / l : 0.0f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const float v4[4] = {acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]};
        store_row<QT, 4>(p.out + (row.qoff + dt * 16 + 4 * kg) * QE, v4, mul);
      }
    }
    return;
  }

  // the last part: its chunk's first part unless it is the run's only one
  const int slot = (pieces == 1 && pos != wstart) ? 1 : 0;
  const RecordRef rec = record_ref<D, R>(p.partials + (int64_t)(2 * last_v + slot) * R * (D + 4));
  mfma_store_record<KV, D>(rec, row.valid && j16 < R, acc, m, l);
  if (arrive(p, first_w, last_w, pieces)) merge_records<QT, D, R>(p, first_w, last_w, seg_start, grid, rows, vs);
}

// Decode: the G query heads of sequence s served by kv head h, one token each.
template <typename KV, typename QT, int D, int G, int POL>
__device__ inline void mfma_run(const DecodeParams& p, int w, const ChunkGrid& grid, int wstart, int pos, int s,
                                int h, int off, int len, int n, int nb) {
  const int Hq = p.num_kv_heads * G;
  const int j16 = threadIdx.x & 15;
  const int64_t orow = ((int64_t)s * Hq + (int64_t)h * G) * D;
  MfmaRow row;
  row.valid = j16 < G;
  row.qoff = orow + (int64_t)j16 * D;
  row.limit = n;
  row.min_limit = n;
  mfma_rows_run<KV, QT, D, G, POL, ContiguousRows, false, true>(p, w, grid, wstart, pos, s, h, off, len, n, nb, row,
                                                                 ContiguousRows{orow, D});
}

}  // namespace pkv
