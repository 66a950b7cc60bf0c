// gemm_tiled.hip -- tiled (prefill) variant of the expert GEMMs.
// Conventions and operand layouts: gemm_common.h.
#include <type_traits>

#include "gemm_common.h"

namespace moe {

// ---------------------------------------------------------------------------
// Tiled variant (prefill): a work item is (expert e, 256 weight rows, BM =
// 16*MT token rows).  Each 64-row weight quad (GEMM1: one gate/up unit) is
// computed by its MFMA waves on all the item's rows, so every weight
// fragment is read from HBM once per item and feeds MT MFMAs; the activation
// tile of a K step is shared by all waves.  Every operand of a K step -- the
// BM activation rows (16-byte chunks XOR-swizzled by row), their E8M0
// scales, each quad's four 1 KiB weight fragments and their scale dword --
// is copied from global memory straight into LDS with global_load_lds (no
// register staging), several steps deep, the copies of a later step
// interleaved with the MFMAs of the current one; the waits count those
// copies exactly (they are the only vector-memory instructions in the loop
// and issue in program order).  BM is picked per call so that most experts
// fit one m-block (each weight panel is then read once).  The logical
// workgroup index is remapped so consecutive items share an XCD and its L2.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void *lds_ptr_t;
typedef __attribute__((address_space(1))) void *glb_ptr_t;

// lane i of the wave copies 16 (4) bytes from its own address g to
// lds_base + 16*i (4*i); lds_base must be wave-uniform
__device__ __forceinline__ void copy16_to_lds(const void *g, void *lds_base) {
  __builtin_amdgcn_global_load_lds((glb_ptr_t)g, (lds_ptr_t)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void copy4_to_lds(const void *g, void *lds_base) {
  __builtin_amdgcn_global_load_lds((glb_ptr_t)g, (lds_ptr_t)lds_base, 4, 0, 0);
}

// s_waitcnt vmcnt(N), expcnt and lgkmcnt left free (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Workgroup barrier for the copy pipeline: LDS reads of this wave done, no
// wait on the copies still in flight (a __syncthreads would wait for all of
// them, since they write LDS).
__device__ __forceinline__ void barrier_keep_copies() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt untouched
  __builtin_amdgcn_s_barrier();
}
// LDS position of the activation tile's 16-byte chunks: chunk c of tile row
// `row` sits at position c ^ act_swizzle(row) of that row.  A wave reads one
// chunk from each of 16 consecutive rows per 16-lane group (the MFMA operand
// of lane group g), so those 16 chunks must fall in different 16-byte bank
// groups of a 256-byte LDS line.  MXFP8 rows are 128 bytes (8 chunks): two
// rows per line, the XOR with the row's low three bits spreads them.  MXFP4
// rows are 64 bytes (4 chunks): four rows per line, rows r and r + 4, r + 8,
// r + 12 share a line position, so the XOR takes bits 2-3 of the row.  (It
// took bits 0-1 before, which vary with the line position itself: 29% of the
// LDS cycles of the A4W4 GEMM1 were bank conflicts.)
template <int FMT>
__device__ __forceinline__ int act_swizzle(int row) {
  return FMT == 0 ? (row & 7) : ((row >> 2) & 3);
}

// Epilogue of one weight quad u of a work item (output tiles 4u .. 4u+3 of
// acc; tile0 the quad's first 16-row weight tile): GEMM1 SwiGLU + requant to
// the A2 rows, GEMM2 weighted rows to the staging buffer.  A padded row
// (loaded from the last valid row) stores the same values as that row, so
// every store is unconditional.
template <class F, int FMT, int MTW, int NT, bool SECOND>
__device__ __forceinline__ void store_item(const KArgs &p, const v4f (&acc)[MTW][NT], int u,
                                           int tile0, int mw0, int row0, int nrows, int g,
                                           int r16) {
  // the row of this lane after a quad transpose (dword-store epilogue)
  auto trow = [&](int m) __attribute__((always_inline)) {
    return (size_t)(row0 + min(16 * (mw0 + m) + 4 * g + (r16 & 3), nrows - 1));
  };
  if (!SECOND) {
    const int j = tile0 / 4;  // unit: h columns [32j, 32j + 32)
    const size_t N = (size_t)p.T * p.top_k;
#pragma unroll
    for (int m = 0; m < MTW; ++m) {
      float g0[4], g1[4], u0[4], u1[4];
      size_t prow[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int mrow = 16 * (mw0 + m) + 4 * g + r;
        prow[r] = (size_t)(row0 + min(mrow, nrows - 1));
        g0[r] = acc[m][4 * u][r]; g1[r] = acc[m][4 * u + 1][r];
        u0[r] = acc[m][4 * u + 2][r]; u1[r] = acc[m][4 * u + 3][r];
      }
      if (FMT == 0) {
        const size_t tr = trow(m);
        swiglu_store_f8_t(g0, g1, u0, u1, p.a2c + a2c_at<0>(tr, j >> 2, N),
                          p.a2s + a2s_at(tr, j >> 2, N), j & 3, r16);
      } else {
        swiglu_requant_n<F, FMT, 4>(g0, g1, u0, u1, p.a2c, p.a2s, prow, N, j, r16);
      }
    }
  } else {
    // the routing weights are loaded per m-tile (all of them at once do not
    // fit the register budget of the producer/consumer form)
#pragma unroll
    for (int m = 0; m < MTW; ++m) {
      size_t prow[4];
      float wa[4], t[4][4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        prow[r] = (size_t)(row0 + min(16 * (mw0 + m) + 4 * g + r, nrows - 1));
        wa[r] = p.wts[prow[r]];
      }
      // the four loads leave together and are waited for once (scheduled
      // next to their uses, each waited for all copies in flight in turn)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q) t[r][q] = wa[r] * acc[m][4 * u + q][r];
      // (a quad-transposed form with one 16-byte store per tile measured
      // 14-22% slower for GEMM2 than these 64-byte row pieces)
      stage_store_n<4>(p, prow, 16 * tile0, r16, t);
    }
  }
}

// ---------------------------------------------------------------------------
// The tiled kernel, in producer/consumer form.  Copy waits count a wave's
// own copies in issue order, so a wave that copied both operands would give
// a step's weights (HBM) and activations (L2) one deadline (an earlier form
// did, and measured 7-8% slower for GEMM1 and 2-6% for GEMM2).  Here the
// consumer waves (RS per weight quad: wave c computes
// quad c % 4 on m-tiles [(c / 4) MT / RS, +MT / RS)) copy only their quad's
// four 1 KiB fragments (a share each) and its scale dword into a ring of NB
// weight stages, NB - 1 steps ahead, and wait only for those; the producer
// waves after them copy the activation tile and its scales into the
// NA-stage activation ring, an equal share each, and wait only for those.
// The barrier of every step makes each wave's copies visible to the others.
// Copies past the last K step re-read a valid step (cache hits) into a ring
// slot no later step reads.
// ---------------------------------------------------------------------------
// Producer waves and ring depths: two producer waves (each with its own
// copy count, so the activation ring can be four stages deep within the
// 63 outstanding copies a wave can wait on) and four stages of each operand
// measured 2% faster per call than one producer with three activation and
// five weight stages on the 7168 x 3072 layer (A8W4 T = 8192, A4W4
// T = 16384) and equal on the 5120 x 640 one; three producers with five
// activation stages, and passing the step barrier before the last m-tile's
// MFMAs, measured no faster.
// Consumer waves: two per weight quad (kPcRowSplit = 2), each with half of
// the item's m-tiles, so two MFMA waves share a SIMD and one issues while
// the other waits on LDS or a copy; measured 3% faster per call at A4W4
// T = 16384 and 2.5% on the 5120 x 640 shard than one wave per quad, equal
// on the 7168 x 3072 layer at A8W4 T = 4096 and 8192.
constexpr int kPcProducers = 2, kPcActStages = 4, kPcWStages = 4, kPcRowSplit = 2;
// Activation scales of GEMM1 (SG): a token row's E8M0 bytes of one K step
// are one dword, so a step's scale copies gather 4 bytes from each of BM
// rows (64 rows, 64 cache lines, per copy), which on this device costs about
// as much per copy as a whole 1 KiB activation chunk.  (GEMM2's scales are
// K-step-major: a step's 64 rows are one 256-byte run.)  Where K / 128 is a
// multiple of four, the copies instead take 16 bytes per row, the scales of
// four K steps (a group), one 64-row part of the next group per step, into
// three rotating group buffers (group g is read in steps 4g .. 4g + 3; its
// parts are issued with steps 4g - 4 .. 4g - 1, so the ring's step wait
// covers them, and the buffer they fill was last read in steps 4g - 12 ..
// 4g - 9, before any of them is issued).  Rows past a part's 64 (BM not a
// multiple of 64, fewer than four parts) repeat the last part: the same
// bytes to the same place.
template <int FMT, int MT, bool SG = false>
struct PcShape {
  static constexpr int NP = kPcProducers;             // producer waves
  static constexpr int RS = kPcRowSplit;              // consumer waves per weight quad
  static constexpr int NC = 4 * RS;                   // consumer waves
  static constexpr int NWAVES = NC + NP;
  static constexpr int MTW = MT / RS;                 // m-tiles per consumer wave
  static constexpr int BM = 16 * MT;
  static constexpr int ROWB = FMT == 0 ? 128 : 64;    // activation bytes per row per K step
  static constexpr int CH = ROWB / 16;
  static constexpr int A_BYTES = BM * ROWB;
  static constexpr int A_CHUNKS = A_BYTES / 1024;     // 1 KiB copies per stage
  static constexpr int SC = (BM + 63) / 64;           // scale copies per stage (64 rows each)
  static constexpr int CA_ALL = A_CHUNKS + (SG ? 1 : SC);  // activation copies per step
  static constexpr int CA = (CA_ALL + NP - 1) / NP;   // per producer wave (the last repeats)
  static constexpr int OFF_AS = A_BYTES;              // [BM] scale dwords (not SG)
  static constexpr int A_STAGE = A_BYTES + (SG ? 0 : 1024);
  static constexpr int GRP = SC * 1024;               // SG: one group buffer, [64 SC rows][16 B]
  static constexpr int NGRP = SG ? 3 : 0;
  static constexpr int CB = 4 / RS + 1;               // consumer copies per step (fragments, scale)
  static constexpr int OFF_BS = 4 * 4096;
  static constexpr int B_STAGE = OFF_BS + 4 * 256;
  // a 192-row MXFP8 tile (24 KiB a stage) keeps three activation stages so
  // that four weight stages still fit
  static constexpr int NA = A_BYTES > 20 * 1024 ? 3 : kPcActStages;
  static constexpr int GRP_BASE = NA * A_STAGE;
  // (the 16 bytes after the rings hold the work-distribution slots)
  static constexpr int NB_FIT = (160 * 1024 - 16 - NA * A_STAGE - NGRP * GRP) / B_STAGE;
  static constexpr int NB = NB_FIT < kPcWStages ? NB_FIT : kPcWStages;
  static constexpr int B_BASE = GRP_BASE + NGRP * GRP;
  static constexpr int LDS = B_BASE + NB * B_STAGE;
  static_assert(A_BYTES % 1024 == 0, "activation tile must fill whole copies");
  static_assert(MT % RS == 0 && 4 % RS == 0, "even row split");
  static_assert(BM <= 256, "scale slots");
  static_assert(NB >= 3, "weight ring");
  static_assert((NA - 1) * CA + 4 < 64 && (NB - 1) * CB < 64, "vmcnt range");
  static_assert(!SG || SC <= 4, "four parts per group");
  static_assert(LDS + 16 <= 160 * 1024, "LDS");
};

template <int FMT, int MT, bool SECOND, bool SG>
__global__ __launch_bounds__(64 * (4 * kPcRowSplit + kPcProducers), 1) void pc_kernel(KArgs p) {
  using F = typename ActFmt<FMT>::F;
  using PS = PcShape<FMT, MT, SG>;
  constexpr int NA = PS::NA, NB = PS::NB, BM = PS::BM, ROWB = PS::ROWB, CH = PS::CH;
  // (one LDS object: the work-distribution slots sit after the rings; a
  // second __shared__ array made the compiler wait for every copy in flight
  // before each LDS read of the MFMA loop)
  __shared__ __attribute__((aligned(16))) uint8_t lds[PS::LDS + 16];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const bool producer = uniform(wave) >= PS::NC;
  const int g = lane >> 4, r16 = lane & 15;
  const int K = SECOND ? p.I : p.H;
  const int S = K / 128;
  const int ntiles = (SECOND ? p.H : 2 * p.I) / 16;
  const int NBLK = (ntiles + 15) / 16;
  const int n_mb = uniform(p.mtoff[p.E]);
  const long total = (long)n_mb * NBLK;
  // A1: token rows (row-major: K step s of a row at s times the step bytes);
  // A2: K-step-major sorted rows (K step s of all N rows one block)
  const size_t arow = FMT == 0 ? (size_t)K : (size_t)K / 2;
  const size_t srow = (size_t)K / 32;
  const size_t NA2 = (size_t)p.T * p.top_k;
  const size_t cstep = SECOND ? NA2 * ROWB : (size_t)ROWB;  // code bytes from a step to the next
  const size_t sstep = SECOND ? NA2 * 4 : 4;                 // scale bytes from a step to the next
  const size_t quad_bytes = (size_t)S * 4096, quad_dwords = (size_t)S * 64;
  const uint8_t *__restrict__ A = SECOND ? p.a2c : p.a1c;
  const uint8_t *__restrict__ As = SECOND ? p.a2s : p.a1s;
  const int G = gridDim.x;
  const int L = (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8);
  const int swz = act_swizzle<FMT>(r16);
  const int aoff_lo = r16 * ROWB + 16 * (g ^ swz);
  const int aoff_hi = r16 * ROWB + 16 * ((4 + g) ^ swz);

  // Consumer weight stream across items (XITEM): the copies of a step NB - 1
  // steps ahead run on from an item's last steps into the next item's first
  // ones (the next item of this workgroup is w + G), so the weights keep
  // streaming through the epilogue and an item never starts on an empty
  // ring.  The ring slot of a step is its position in this workgroup's whole
  // sequence of steps, modulo NB.  Past the last item the copies re-read a
  // valid step into slots no step reads.  It measured 1.5% faster per call
  // (A4W4, T = 16384, MT = 8); at MT = 10 its extra live registers spill, so
  // there each item issues its own first NB - 1 steps and its copies past
  // the last step re-read that step.  (With two consumer waves per quad a
  // wave holds MT / 2 m-tiles, and the cross-item stream runs at every tile
  // height up to 160 rows; at 192 rows (6 m-tiles a wave) its registers
  // would spill, so there each item issues its own first steps.)
  constexpr bool XITEM = MT / kPcRowSplit <= 5;
  // Work distribution.  The list is dealt to the eight XCDs in chunks of G / 8
  // consecutive items, chunk j to XCD j % 8 (the order a fixed stride of G
  // gives: the whole device works on neighbouring items), and the workgroups
  // of XCD x (b % 8 == x: the hardware deals workgroups to the XCDs in turn)
  // take XCD x's items in order from the XCD's own counter, one at a time:
  // whatever their timing, the workgroups of one XCD work on neighbouring
  // items (one expert's m-blocks and n-blocks), so the m-blocks that read one
  // weight panel run together and find it in the XCD's L2.  (With each
  // workgroup on a fixed stride of G items, workgroups that started together
  // on two m-blocks of one panel drifted apart over the rounds.)  Workgroup
  // item k is taken at the start of item k - 1 by the first producer wave
  // and passed on in LDS; the weight cursor needs item k + 1 from step
  // S - NB + 1 of item k on, so counters are used when S >= NB (every
  // measured shape), else the fixed stride.
  int *const qslot = reinterpret_cast<int *>(lds + PS::LDS);
  const bool dyn = !SECOND && S >= NB;
  const int xcd = (int)(blockIdx.x % 8);
  const int qchunk = G / 8;
  int *const qctr = p.sync + kQueueBase + (SECOND ? 8 : 0) + xcd;
  // the c-th item of XCD x's sequence (total when past the list's end)
  auto xcd_item = [&](int c) __attribute__((always_inline)) {
    const long w = ((long)(c / qchunk) * 8 + xcd) * qchunk + c % qchunk;
    return w < total ? (int)w : (int)total;
  };
  const int qd = uniform(wave & 3);  // the weight quad a consumer wave computes and copies
  const int rh = PS::RS == 1 ? 0 : uniform(wave >> 2);  // its share of the copies and m-tiles
  constexpr int MTW = PS::MTW;
  const int total_i = (int)total;      // items fit 32 bits (m-blocks x n-blocks)
  // this workgroup's item k, given its item k - 1 (items at or past total_i:
  // none left)
  auto next_item = [&](int wprev, int k) __attribute__((always_inline)) {
    return dyn ? uniform(qslot[k & 3]) : wprev + G;
  };
  if (dyn) {
    if (tid == 0) qslot[0] = xcd_item(atomicAdd(qctr, 1));
    __syncthreads();
  }
  // Item wi of the list: the items of expert e are [NBLK mtoff[e], NBLK
  // mtoff[e+1]), n-block major and m-block minor, so the m-blocks that read
  // one weight panel are consecutive items: they run at the same time on
  // neighbouring workgroups of one XCD (see L above), and all but the first
  // find the panel in that XCD's L2.  (With the m-block-major order an
  // expert's second m-block read its panels again from HBM, NBLK items later
  // and usually on another XCD.)
  auto coords = [&](int wi, int &ei, int &nbi, int &mbi) __attribute__((always_inline)) {
    ei = uniform(p.mbexp[wi / NBLK]);
    const int m0 = uniform(p.mtoff[ei]), nmb = uniform(p.mtoff[ei + 1]) - m0;
    const int i = wi - NBLK * m0;
    nbi = uniform(i / nmb);
    mbi = uniform(i - nbi * nmb);
  };
  auto quad_of = [&](int wi) __attribute__((always_inline)) {
    int ei, nbi, mbi;
    coords(wi, ei, nbi, mbi);
    const int ti = 16 * nbi + 4 * qd;  // quads past the last tile read quad 0
    return uniform(ei * (ntiles / 4) + (ti < ntiles ? ti / 4 : 0));
  };
  int ck = 0;                                // this workgroup's index of the item of the next copy
  int cw = dyn ? uniform(qslot[0]) : L;      // that item
  int cs = 0;                                // its step
  int cslot = 0;                             // its ring slot
  int cqb = cw < total_i ? quad_of(cw) : 0;
  int rslot = 0;      // ring slot of the current item's step 0
  // weight copy i of the cursor's step
  auto issue_next = [&](int i) __attribute__((always_inline)) {
    const int sr = cw < total_i ? cs : S - 1;
    uint8_t *sw = lds + PS::B_BASE + cslot * PS::B_STAGE;
    // a wave-uniform base plus a 32-bit lane offset (the scalar-base form of
    // the copy: no 64-bit address per lane)
    // the 4 / RS fragments of this wave's share, then the quad's scale
    // dword (each wave of a quad copies it: same bytes, same LDS address)
    const int f = rh * (4 / PS::RS) + i;
    if (i < 4 / PS::RS) {
      // (copying these with the non-temporal hint measured 4% faster per call
      // where each expert is one m-block, 5-14% slower where later m-blocks
      // re-read the panels from L2, and a run-time choice between the two
      // forms cost 11% through code generation at 160 rows: not used)
      copy16_to_lds(p.wp + ((size_t)cqb * quad_bytes + (size_t)sr * 4096) +
                        (uint32_t)(f * 1024 + lane * 16),
                    sw + (4 * qd + f) * 1024);
    } else if (rh == 0) {
      // the quad's scale dword: one wave of the quad copies it (the barrier of
      // the step makes it visible to the other)
      copy4_to_lds(reinterpret_cast<const uint8_t *>(p.wsp + (size_t)cqb * quad_dwords +
                                                     (size_t)sr * 64) +
                       (uint32_t)(lane * 4),
                   sw + PS::OFF_BS + qd * 256);
    }
  };
  // the wait for the copies of the step NB - 2 steps behind the cursor: the
  // wave with rh == 0 issues CB copies per step (its fragments and the scale
  // dword), the others CB - 1
  auto wait_weights = [&]() __attribute__((always_inline)) {
    if (rh == 0)
      wait_vm<(NB - 2) * PS::CB>();
    else
      wait_vm<(NB - 2) * (PS::CB - 1)>();
  };
  // the cursor moves to the next step once all its copies are issued
  auto advance = [&]() __attribute__((always_inline)) {
    cslot = cslot + 1 == NB ? 0 : cslot + 1;
    if (++cs == S) {
      if (XITEM) {
        cs = 0;
        cw = next_item(cw, ++ck);
        if (cw < total_i) cqb = quad_of(cw);
      } else {
        cs = S - 1;  // re-read the last step until the next item starts
      }
    }
  };
  if (XITEM && !producer) {
#pragma unroll
    for (int st = 0; st < NB - 1; ++st) {
#pragma unroll
      for (int i = 0; i < PS::CB; ++i) issue_next(i);
      advance();
    }
  }

  for (int k = 0, w = dyn ? uniform(qslot[0]) : L; w < total_i; w = next_item(w, ++k)) {
    int e, nb, mb;
    coords(w, e, nb, mb);
    const int row0 = uniform(p.offsets[e]) + BM * mb;
    const int nrows = min(BM, uniform(p.offsets[e + 1]) - row0);

    if (producer) {
      // producer wave PW issues copies [PW * CA, PW * CA + CA) of a step's
      // CA_ALL (activation chunks, then scale dwords); an index past the last
      // repeats the last copy (same bytes to the same LDS address)
      auto produce = [&](auto pwc) __attribute__((always_inline)) {
        constexpr int PW = decltype(pwc)::value;
        // copy index c of this wave: activation chunk i < A_CHUNKS, else a
        // scale copy; an index past the last repeats a copy (SG: the last
        // chunk, so that the group part is issued once per step)
        auto copy_index = [&](int c) __attribute__((always_inline)) {
          return PW * PS::CA + c < PS::CA_ALL ? PW * PS::CA + c
                                             : (SG ? PS::A_CHUNKS - 1 : PS::CA_ALL - 1);
        };
        // SG: the wave issuing the group parts, and the offset of each part's
        // row for this lane in 16-byte units (rows are whole units under SG)
        constexpr bool GW = SG && PW * PS::CA <= PS::A_CHUNKS && PS::A_CHUNKS < PW * PS::CA + PS::CA;
        uint32_t gro[4];
        if (GW) {
#pragma unroll
          for (int part = 0; part < 4; ++part) {
            const int row = min(64 * min(part, PS::SC - 1) + lane, BM - 1);
            const int rr = min(row, nrows - 1);
            const size_t ridx =
                SECOND ? (size_t)(row0 + rr) : (size_t)(p.perm[row0 + rr] / p.top_k);
            gro[part] = (uint32_t)(ridx * (srow / 16));
          }
        }
        // part `part` of group gi (data of group min(gi, last)) into its buffer
        auto issue_group = [&](int part, int gi) __attribute__((always_inline)) {
          const int gd = min(gi, S / 4 - 1);
          const uint32_t ro = part == 0 ? gro[0] : part == 1 ? gro[1] : part == 2 ? gro[2] : gro[3];
          copy16_to_lds(As + 16 * ((size_t)ro + gd),
                        lds + PS::GRP_BASE + (gi % 3) * PS::GRP + 1024 * min(part, PS::SC - 1));
        };
        const uint8_t *csrc[PS::CA];
#pragma unroll
        for (int c = 0; c < PS::CA; ++c) {
          const int i = copy_index(c);
          const bool chunk = i < PS::A_CHUNKS;
          const int ci = i * 64 + lane;  // 16-byte LDS chunk this lane fills
          const int row = chunk ? ci / CH : min(64 * (i - PS::A_CHUNKS) + lane, BM - 1);
          const int rr = min(row, nrows - 1);
          const size_t ridx =
              SECOND ? (size_t)(row0 + rr) : (size_t)(p.perm[row0 + rr] / p.top_k);
          csrc[c] = chunk ? A + ridx * (SECOND ? (size_t)ROWB : arow) +
                                16 * ((ci % CH) ^ act_swizzle<FMT>(row))
                          : As + ridx * (SECOND ? (size_t)4 : srow);
        }
        // the first producer takes this workgroup's next item, after the row
        // gathers above (its reply is older than the first stages' copies, so
        // their wait covers it)
        int taken = 0;
        if (PW == 0 && dyn && lane == 0) taken = atomicAdd(qctr, 1);
        auto issue_a = [&](int st) __attribute__((always_inline)) {
          const int sr = min(st, S - 1);
          uint8_t *stg = lds + (st % NA) * PS::A_STAGE;
#pragma unroll
          for (int c = 0; c < PS::CA; ++c) {
            const int i = copy_index(c);
            if (i < PS::A_CHUNKS)
              copy16_to_lds(csrc[c] + cstep * sr, stg + i * 1024);
            else if (SG)
              issue_group(st & 3, (st >> 2) + 1);  // part st % 4 of the next group
            else
              copy4_to_lds(csrc[c] + sstep * sr, stg + PS::OFF_AS + 256 * (i - PS::A_CHUNKS));
          }
        };
        // SG: group 0 before the first steps (older than step 0's copies, so
        // the wait for step 0 covers it)
        if (GW) {
#pragma unroll
          for (int part = 0; part < PS::SC; ++part) issue_group(part, 0);
        }
#pragma unroll
        for (int st = 0; st < NA - 1; ++st) issue_a(st);
        wait_vm<(NA - 2) * PS::CA>();  // step 0 has landed
        if (PW == 0 && dyn && lane == 0) qslot[(k + 1) & 3] = xcd_item(taken);
        barrier_keep_copies();
        for (int s = 0; s < S; ++s) {
          issue_a(s + NA - 1);
          wait_vm<(NA - 2) * PS::CA>();  // step s+1 has landed
          barrier_keep_copies();
        }
      };
      if (PS::NP == 1 || wave == PS::NC)
        produce(std::integral_constant<int, 0>{});
      else if (PS::NP == 2 || wave == PS::NC + 1)
        produce(std::integral_constant<int, PS::NP >= 2 ? 1 : 0>{});
      else
        produce(std::integral_constant<int, PS::NP >= 3 ? 2 : 0>{});
      wait_vm<0>();
    } else {
      const int t0 = 16 * nb + 4 * qd;
      auto read_a = [&](const uint8_t *st, int m) __attribute__((always_inline)) {
        v8i a;
        const uint8_t *base = st + m * 16 * ROWB;
        const u32x4 lo = *reinterpret_cast<const u32x4 *>(base + aoff_lo);
        a[0] = (int)lo[0]; a[1] = (int)lo[1]; a[2] = (int)lo[2]; a[3] = (int)lo[3];
        if (FMT == 0) {
          const u32x4 hi = *reinterpret_cast<const u32x4 *>(base + aoff_hi);
          a[4] = (int)hi[0]; a[5] = (int)hi[1]; a[6] = (int)hi[2]; a[7] = (int)hi[3];
        } else {
          a[4] = 0; a[5] = 0; a[6] = 0; a[7] = 0;
        }
        return a;
      };
      // the scale byte of this lane's row and block g: st is the step's stage
      // (its scale dwords), or with SG the step's dword column of its group
      // buffer
      auto read_sa = [&](const uint8_t *st, int m) __attribute__((always_inline)) {
        return SG ? (int)st[16 * (16 * m + r16) + g] : (int)st[PS::OFF_AS + 4 * (16 * m + r16) + g];
      };
      if (!XITEM) {
        cw = w;
        cs = 0;
        cqb = quad_of(w);
        rslot = cslot;
#pragma unroll
        for (int st = 0; st < NB - 1; ++st) {
#pragma unroll
          for (int i = 0; i < PS::CB; ++i) issue_next(i);
          advance();
        }
      }
      // step 0's copies were issued NB - 1 steps ago (with XITEM: in the last
      // steps of the previous item, or before the first; the previous
      // epilogue's stores, issued after them, also drain here)
      wait_weights();  // step 0 has landed
      barrier_keep_copies();

      // the MFMA loop and epilogue of this wave's m-tiles, compiled once per
      // row half so that the m-tile offset is a constant in every address
      auto consume = [&](auto rhc) __attribute__((always_inline)) {
        constexpr int MW0 = decltype(rhc)::value * MTW;
        v4f acc[MTW][4];
  #pragma unroll
        for (int m = 0; m < MTW; ++m)
  #pragma unroll
          for (int q = 0; q < 4; ++q) acc[m][q] = v4f{0.f, 0.f, 0.f, 0.f};
        // the weight fragments and scale dword of K step st
        auto read_b = [&](int slot, v8i (&bb)[4], int &sbb) __attribute__((always_inline)) {
          const uint8_t *sw = lds + PS::B_BASE + slot * PS::B_STAGE;
          sbb = *reinterpret_cast<const int *>(sw + PS::OFF_BS + qd * 256 + lane * 4);
  #pragma unroll
          for (int q = 0; q < 4; ++q) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(sw + qd * 4096 + q * 1024 + lane * 16);
            bb[q][0] = (int)v[0]; bb[q][1] = (int)v[1]; bb[q][2] = (int)v[2]; bb[q][3] = (int)v[3];
            bb[q][4] = 0; bb[q][5] = 0; bb[q][6] = 0; bb[q][7] = 0;
          }
        };
        for (int s = 0; s < S; ++s) {
          const uint8_t *st = lds + (s % NA) * PS::A_STAGE;
          const uint8_t *ss =
              SG ? lds + PS::GRP_BASE + ((s >> 2) % 3) * PS::GRP + 4 * (s & 3) : st;
          int sb;
          v8i b[4];
          read_b(rslot, b, sb);
          rslot = rslot + 1 == NB ? 0 : rslot + 1;
          v8i acur = read_a(st, MW0);
          int sacur = read_sa(ss, MW0);
  #pragma unroll
          for (int m = 0; m < MTW; ++m) {
  #pragma unroll
            for (int i = m * PS::CB / MTW; i < (m + 1) * PS::CB / MTW; ++i) issue_next(i);
            v8i anext = acur;
            int sanext = sacur;
            if (m + 1 < MTW) {
              anext = read_a(st, MW0 + m + 1);
              sanext = read_sa(ss, MW0 + m + 1);
            }
  #pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[m][q] = mfma_q<FMT>(q, acur, b[q], acc[m][q], sacur, sb);
            __builtin_amdgcn_sched_barrier(0);
            acur = anext;
            sacur = sanext;
          }
          __builtin_amdgcn_sched_barrier(0);
          advance();
          wait_weights();  // step s+1's weights have landed
          barrier_keep_copies();
        }
        // without XITEM the re-reads past the last step land before the next
        // item's first copies reuse their slots
        if (!XITEM) wait_vm<0>();
        if (t0 < ntiles) store_item<F, FMT, MTW, 4, SECOND>(p, acc, 0, t0, MW0, row0, nrows, g, r16);
      };
      if (PS::RS == 1 || rh == 0)
        consume(std::integral_constant<int, 0>{});
      else
        consume(std::integral_constant<int, PS::RS >= 2 ? 1 : 0>{});
    }
  }
  wait_vm<0>();  // no copy into this workgroup's LDS outlives it
}

template <bool SECOND, bool SG>
static hipError_t launch_pc(const GemmArgs &a, const KArgs &k, hipStream_t s) {
  const unsigned grid = (unsigned)(a.num_cus / 8 * 8);  // one workgroup per CU
#define PC(F_, MT_)                                          \
  case MT_:                                                  \
    pc_kernel<F_, MT_, SECOND, SG><<<grid, 64 * PcShape<F_, MT_, SG>::NWAVES, 0, s>>>(k); \
    break;
  if (a.act == MOE_ACT_MXFP8_E4M3) {
    switch (a.plan.mt) {
      PC(0, 2) PC(0, 4) PC(0, 6) PC(0, 8) PC(0, 10) PC(0, 12)
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (a.plan.mt) {
      PC(4, 2) PC(4, 4) PC(4, 6) PC(4, 8) PC(4, 10) PC(4, 12)
      default: return hipErrorInvalidValue;
    }
  }
#undef PC
  return hipGetLastError();
}

template <bool SECOND>
static hipError_t launch_tiled(const GemmArgs &a, const KArgs &k, hipStream_t s) {
  if (a.plan.split != kTiledSplit) return hipErrorInvalidValue;
  // GEMM2's scales are K-step-major (a step's rows contiguous): no groups
  if constexpr (SECOND) {
    return launch_pc<true, false>(a, k, s);
  } else {
    // scale groups: whole groups of four K steps, and 16-byte aligned rows;
    // not at 192 MXFP8 rows, where the group addresses made the kernel spill
    // registers (2-5% slower per call on the 5120 x 640 shard at T = 32768)
    const bool sg = (a.H / 128) % 4 == 0 && reinterpret_cast<uintptr_t>(a.a1s) % 16 == 0 &&
                    !(a.act == MOE_ACT_MXFP8_E4M3 && a.plan.mt == 12);
    return sg ? launch_pc<false, true>(a, k, s) : launch_pc<false, false>(a, k, s);
  }
}

hipError_t launch_tiled_gemm1(const GemmArgs &a, const KArgs &k, hipStream_t s) {
  return launch_tiled<false>(a, k, s);
}

hipError_t launch_tiled_gemm2(const GemmArgs &a, const KArgs &k, hipStream_t s) {
  return launch_tiled<true>(a, k, s);
}

}  // namespace moe
