#pragma once
// gemm_nv.hpp -- NVFP4 prefill schedule with the activation operand
// dequantized once per workgroup (part of gemm_kernels.hpp; FlashRT fp4-gemm
// README, "Available Functions": nvfp4_gemm_bf16 and its epilogues, on
// NVFP4 operands with E4M3 16-element block scales).
//
// Why a second NVFP4 prefill schedule.  NVFP4 reaches the fp16 MFMA through
// an exact per-element dequantization (FP4 -> fp16 conversion with the scale's
// power of two, then one packed multiply by its mantissa).  On gfx950 the
// conversion issues at about 9 cycles a wave instruction, twice the cost of
// the packed multiply, and only about two conversions hide under one 32-cycle
// fp16 MFMA.  When every wave converts all of its own operands (4 x 3
// fragments per 12 MFMAs) the schedule is bound by that work.  Here the tile is
// 128 A rows x 384 B columns; wave w owns columns [96w, 96w + 96) (4 x 3
// accumulator tiles of 32 x 32).  Each wave converts its own 3 B fragments,
// but the 4 A fragments, which all four waves use, are converted once per
// workgroup: wave w converts A fragment w and writes it to LDS, where every
// wave reads it.  A wave then converts 1/3 of a fragment
// per MFMA instead of 7/12.  The LDS exchange moves 32 KiB of writes and
// 96 KiB of reads per workgroup and stage, about 40% of what LDS delivers in
// the MFMAs' time.  Measured on the chain's shapes it is 5-8% faster than the
// 256 x 192 schedule: a wave still issues 12 MFMAs a step behind one
// in-order instruction stream with about 240 cycles of conversion work, and
// the operand loads cost about as much again as the ideal overlap leaves.
//
// K order.  K runs in stages of 128 elements (64 bytes of a packed row).
// Lane (r, c) of a fragment (r = lane % 32 the row, c = lane / 32) covers the
// stage's elements [64c, 64c + 64): K16 step t takes elements 64c + 8t .. + 7,
// the lane's dword t.  Both operands use this order, so the contraction is
// unchanged.  The lane's four blocks, 8s + 4c .. + 3 of stage s (step t uses
// the block t / 2 among them), are one 32-bit scale word in either layout:
// LINEAR bytes row * nblk + 8s + 4c (nblk % 4 == 0), TILED word c * 32 + row % 32
// of the row group's 256-byte group s.
//
// Pipeline.  The packed bytes and scale words go straight from memory to
// registers (no LDS staging), two stages ahead, in three rotating register
// sets: 12 loads a wave and stage (16 bytes a lane for the packed bytes),
// spread over the stage's first four steps, one per MFMA -- issued together
// they fill the texture unit's queues and stall the wave.  In stage s a wave
// runs 8 steps of 12 MFMAs; under them it reads the next step's A fragments
// from LDS, converts the next step's B fragments, and converts and writes its
// A fragment's 8 steps of stage s + 1 into the other LDS buffer.  One barrier
// per stage, before its last step, publishes those (and frees the buffer of
// stage s - 1, whose last reads came before it).
//
// Included by gemm_kernels.hpp inside namespace lowbit::gk, after the
// helpers it uses (dq8, NvPart, epi_wave, fp4_out_padding, wait_vm_le_lgkm0).

constexpr int kNvBM = 128, kNvBN = 384, kNvTI = 4, kNvTJ = 3, kNvSteps = 8;
constexpr int kNvUnit = 1024;                              // one fragment step: 64 lanes x 16 B
constexpr int kNvStageLds = kNvSteps * kNvTI * kNvUnit;    // 32 KiB of converted A per stage
constexpr int kNvEpiLds = 4 * 32 * kEpiRowPitch * 4;       // the epilogue's staging, 4 waves
constexpr int kNvLds = (2 * kNvStageLds > kNvEpiLds) ? 2 * kNvStageLds : kNvEpiLds;

struct NvB {                // one stage of a wave's B operand
  u32x4 q[kNvTJ][2];        // the lane's 32 bytes of each fragment
  uint32_t s[kNvTJ];        // its scale word (blocks 8s + 4c .. + 3)
};
struct NvA {                // this wave's share of one stage of A: fragment w
  u32x4 q[2];               // the lane's 32 bytes of it
  uint32_t s;               // its scale word
};

// Power of two and mantissa of E4M3 scale byte (word >> 8 * byte) & 0xFF
// (the split nv_part makes; a zero or absent scale gives p = 0).
__device__ __forceinline__ NvPart nv_part_word(uint32_t word) {
  const float s = __builtin_amdgcn_cvt_f32_fp8((int)word, 0);
  const uint32_t u = __float_as_uint(s);
  const _Float16 h = (_Float16)__uint_as_float((u & 0x807FFFFFu) | 0x3F800000u);
  return NvPart{__uint_as_float(u & 0x7F800000u), v2h{h, h}};
}

// SPLIT: split-K -- workgroup (tile, y) takes stages [y * g.per, (y + 1) * g.per)
// of K and writes its fp32 partial 32 x 32 tiles to the workspace in the
// decode schedule's partial layout (lane (r, c) holds output row r and
// columns 8(k / 4) + 4c + k % 4, 16 floats a lane, tile (y, n / 32, m / 32) at
// ((y * ceil(N / 32) + n / 32) * ceil(M / 32) + m / 32) * 1024 floats), which
// gemm_splitk_reduce_kernel sums in split order before the epilogue.
template <int FMT, int EPI, bool LA_TILED, bool LB_TILED, bool SPLIT = false>
__global__ __launch_bounds__(256, 1) void gemm_prefill_nv_kernel(GemmArgs g) {
  constexpr int TI = kNvTI, TJ = kNvTJ;
  static_assert(FMT == kNVFP4, "NVFP4 operands");
  constexpr int kSteps = kNvSteps;                           // K16 steps of a 64-byte row stage
  constexpr int kStageLds = kSteps * TI * kNvUnit;           // converted A of one stage
  using VT = v8h;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kNvLds];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 31, c = lane >> 5;

  // tile order: consecutive workgroups go to different XCDs, each XCD taking
  // a contiguous eighth of the sequence; groups of 8 M-tiles share B tiles
  const int64_t tiles_m = (g.M + kNvBM - 1) / kNvBM, tiles_n = (g.N + kNvBN - 1) / kNvBN;
  const int64_t T = tiles_m * tiles_n;
  int64_t t = blockIdx.x;
  if (T % 8 == 0) t = (t % 8) * (T / 8) + t / 8;
  const int64_t group = 8 * tiles_n;
  const int64_t first_m = (t / group) * 8;
  const int64_t gsz = (tiles_m - first_m) < 8 ? (tiles_m - first_m) : 8;
  const int64_t tm = first_m + (t % group) % gsz;
  const int64_t tn = (t % group) / gsz;
  const int m0 = (int)(tm * kNvBM), n0 = (int)(tn * kNvBN);

  const int M = (int)g.M, N = (int)g.N;
  const int kbytes = (int)(g.K / 2);                         // packed bytes of a row
  const int nblk = (int)(g.K / 16);
  const int ktiles = (nblk + 7) >> 3;
  const int nst_all = (kbytes + 63) / 64;                    // 64-byte row stages
  const int s0 = SPLIT ? (int)blockIdx.y * g.per : 0;                        // this workgroup's stages
  const int nst = SPLIT ? min(g.per, nst_all - s0) : nst_all;                  // (count)
  const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc((void*)g.a, (short)0, M * kbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc((void*)g.b, (short)0, N * kbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rssa = __builtin_amdgcn_make_buffer_rsrc(
      (void*)g.sfa, (short)0, (int)sf_bytes_of(g.la, g.M, nblk), 0x00020000);
  const __amdgpu_buffer_rsrc_t rssb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)g.sfb, (short)0, (int)sf_bytes_of(g.lb, g.N, nblk), 0x00020000);
  constexpr int kAbsent = 0x40000000;   // beyond every operand buffer (checked by the host)

  // per-lane offsets; the stage advance goes into the scalar offset
  auto sf_base = [&](int row, int R, bool tiled) {
    if (row >= R) return kAbsent;
    return tiled ? (((row >> 5) * ktiles) << 8) + ((c * 32 + (row & 31)) << 2) : row * nblk + 4 * c;
  };
  int ob[TJ], sb_[TJ];
#pragma unroll
  for (int j = 0; j < TJ; j++) {
    const int row = n0 + wave * (TJ * 32) + j * 32 + r;
    ob[j] = row < N ? row * kbytes + 32 * c : kAbsent;
    sb_[j] = sf_base(row, N, LB_TILED);
  }
  const int arow = m0 + wave * 32 + r;   // this wave's A fragment
  const int oa = arow < M ? arow * kbytes + 32 * c : kAbsent;
  const int sa_ = sf_base(arow, M, LA_TILED);
  // part p of stage s's loads into register sets b, a (p = 0: the A fragment;
  // p = 1..3: B fragment p - 1), three loads each.  Only the per-lane offset
  // is range-checked against the buffer, so a stage wholly inside K (every
  // stage but possibly the last) puts its advance in the scalar offset, and
  // the stages at and past the end of K (the last one when K % 128 == 64,
  // and the two issued past the end) put the whole offset in the lane's and
  // turn half-rows beyond K into absent ones (zero bytes, zero scales).  The
  // choice is a select, not a branch: loads in one basic block keep the
  // compiler's waits on their registers exact.
  const int nfull = kbytes / 64;   // stages wholly inside K
  auto issue = [&](int s, int p, NvB& b, NvA& a) {
    const bool fast = s < nfull;                       // uniform
    const int so = s * 64;
    const int ssf = (p == 0 ? LA_TILED : LB_TILED) ? (s << 8) : (s << 3);
    const int sd = fast ? so : 0, ss = fast ? ssf : 0;   // scalar parts
    const int vd = fast ? 0 : so, vs = fast ? 0 : ssf;   // lane parts
    // K % 64 == 0: a lane half is wholly in or out
    const bool in = fast || so + 32 * c < kbytes;
    auto voff = [&](int base, int add) { return in ? base + add : kAbsent; };
    if (p == 0) {
      a.q[0] = __builtin_amdgcn_raw_buffer_load_b128(rsa, voff(oa, vd), sd, 0);
      a.q[1] = __builtin_amdgcn_raw_buffer_load_b128(rsa, voff(oa + 16, vd), sd, 0);
      a.s = __builtin_amdgcn_raw_buffer_load_b32(rssa, voff(sa_, vs), ss, 0);
    } else {
      const int j = p - 1;
      b.q[j][0] = __builtin_amdgcn_raw_buffer_load_b128(rsb, voff(ob[j], vd), sd, 0);
      b.q[j][1] = __builtin_amdgcn_raw_buffer_load_b128(rsb, voff(ob[j] + 16, vd), sd, 0);
      b.s[j] = __builtin_amdgcn_raw_buffer_load_b32(rssb, voff(sb_[j], vs), ss, 0);
    }
  };

  v16f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; i++)
#pragma unroll
    for (int j = 0; j < TJ; j++) acc[i][j] = v16f{};

  // step t of a lane's 32 bytes, dequantized: dword t with the E4M3 scale of
  // block t / 2 (byte t / 2 of the word)
  auto deq = [&](const u32x4 (&q)[2], uint32_t sw, int t, int s) -> VT {
    (void)s;
    return dq8(q[t >> 2][t & 3], nv_part_word(sw >> (8 * (t >> 1))));
  };
  // step t of this wave's A fragment of stage s, dequantized into LDS unit (t, w)
  auto unit = [&](const NvA& a, int t, int s, uint8_t* buf) {
    *reinterpret_cast<VT*>(buf + (t * TI + wave) * kNvUnit + lane * 16) = deq(a.q, a.s, t, s);
  };
  auto read_a = [&](VT (&va)[TI], const uint8_t* buf, int step) {
#pragma unroll
    for (int i = 0; i < TI; i++) va[i] = *reinterpret_cast<const VT*>(buf + (step * TI + i) * kNvUnit + lane * 16);
  };
  auto conv_b = [&](VT (&vb)[TJ], const NvB& b, int step, int s) {
#pragma unroll
    for (int j = 0; j < TJ; j++) vb[j] = deq(b.q[j], b.s[j], step, s);
  };
  auto mma = [&](const VT (&va)[TI], const VT (&vb)[TJ]) {
#pragma unroll
    for (int i = 0; i < TI; i++)
#pragma unroll
      for (int j = 0; j < TJ; j++) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[i], vb[j], acc[i][j], 0, 0, 0);
  };
  // one MFMA, then a share of the VALU work, then one LDS access (the first
  // NDS MFMAs) or one load (the next NVM)
  auto interleave = [&](auto nds, auto nvm) {
    constexpr int NDS = decltype(nds)::value, NVM = decltype(nvm)::value;
#pragma unroll
    for (int k = 0; k < TI * TJ; k++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // VALU
      if (k < NDS) __builtin_amdgcn_sched_group_barrier(0x080, 1, 0);              // one LDS access
      else if (k < NDS + NVM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one load
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I3 = std::integral_constant<int, 3>;

  NvB B0, B1, B2;
  NvA A0, A1, A2;
  VT va[TI], vb[TJ], na[TI], nb[TJ];
  // prologue: stages 0 and 1 in flight; stage 0's A fragment converted and
  // published; step 0 of stage 0 ready in registers
#pragma unroll
  for (int p = 0; p < 4; p++) issue(s0, p, B0, A0);
#pragma unroll
  for (int p = 0; p < 4; p++) issue(s0 + 1, p, B1, A1);
#pragma unroll
  for (int t = 0; t < kSteps; t++) unit(A0, t, s0, smem);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  read_a(va, smem, 0);
  conv_b(vb, B0, 0, s0);

  // the workgroup's stage ls (K stage s0 + ls) from register sets (bc: that
  // stage, bn: the next, bf: the load target two ahead; an: A of the next
  // stage, af: A load target); LDS buffer ls % 2 holds its converted A
  auto stage = [&](int ls, const NvB& bc, const NvB& bn, NvB& bf, const NvA& an, NvA& af) {
    const int s = s0 + ls;
    uint8_t* cur = smem + (ls & 1) * kStageLds;
    uint8_t* nxt = smem + ((ls & 1) ^ 1) * kStageLds;
    // the four load parts of stage s + 2 go out over the first steps, at most
    // one part (three loads) per step where there are steps enough
    constexpr int kLoadSteps = kSteps - 1 < 4 ? kSteps - 1 : 4;
#pragma unroll
    for (int st = 0; st < kSteps - 1; st++) {
      __builtin_amdgcn_sched_barrier(0);
      read_a(na, cur, st + 1);
      conv_b(nb, bc, st + 1, s);
      unit(an, st, s + 1, nxt);
      if (st == kSteps - 2) unit(an, st + 1, s + 1, nxt);
      int nparts = 0;
#pragma unroll
      for (int p = 0; p < 4; p++)
        if (p * kLoadSteps / 4 == st) {
          issue(s + 2, p, bf, af);
          nparts++;
        }
      mma(va, vb);
      if (st == kSteps - 2) {
        if (nparts == 1) interleave(std::integral_constant<int, TI + 2>{}, I3{});
        else interleave(std::integral_constant<int, TI + 2>{}, I0{});
      } else if (nparts == 2) {
        interleave(std::integral_constant<int, TI + 1>{}, std::integral_constant<int, 6>{});
      } else if (nparts == 1) {
        interleave(std::integral_constant<int, TI + 1>{}, I3{});
      } else {
        interleave(std::integral_constant<int, TI + 1>{}, I0{});
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < TI; i++) va[i] = na[i];
#pragma unroll
      for (int j = 0; j < TJ; j++) vb[j] = nb[j];
    }
    // publish stage s + 1's A units; every wave's reads of stage s are done
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_a(na, nxt, 0);
    conv_b(nb, bn, 0, s + 1);
    mma(va, vb);
    interleave(std::integral_constant<int, TI>{}, I0{});
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < TI; i++) va[i] = na[i];
#pragma unroll
    for (int j = 0; j < TJ; j++) vb[j] = nb[j];
  };
  int ls = 0;
  for (; ls + 3 <= nst; ls += 3) {
    stage(ls, B0, B1, B2, A1, A2);
    stage(ls + 1, B1, B2, B0, A2, A0);
    stage(ls + 2, B2, B0, B1, A0, A1);
  }
  if (ls < nst) stage(ls, B0, B1, B2, A1, A2);
  if (ls + 1 < nst) stage(ls + 1, B1, B2, B0, A2, A0);
  // the loads issued past the end land before the epilogue reuses LDS
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
  __syncthreads();

  float* const et = reinterpret_cast<float*>(smem) + wave * 32 * kEpiRowPitch;
  if constexpr (SPLIT) {
    // each row block through LDS, read back transposed into the partial layout
    const int64_t tiles32 = (g.N + 31) / 32, mt = (g.M + 31) / 32;
    auto fence = [&]() {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
#pragma unroll
    for (int i = 0; i < TI; i++) {
      if (m0 / 32 + i >= mt) break;   // uniform: M-tiles past M hold no rows
#pragma unroll
      for (int j = 0; j < TJ; j++)
#pragma unroll
        for (int k = 0; k < 16; k++)
          et[((k >> 2) * 8 + c * 4 + (k & 3)) * kEpiRowPitch + j * 32 + r] = acc[i][j][k];
      fence();
#pragma unroll
      for (int j = 0; j < TJ; j++) {
        const int64_t t32 = (n0 + wave * TJ * 32 + j * 32) / 32;
        if (t32 < tiles32) {
          float4* dst = reinterpret_cast<float4*>(
              g.ws + (((int64_t)blockIdx.y * tiles32 + t32) * mt + m0 / 32 + i) * 1024 + lane * 16);
#pragma unroll
          for (int q = 0; q < 4; q++)
            dst[q] = *reinterpret_cast<const float4*>(et + r * kEpiRowPitch + j * 32 + q * 8 + c * 4);
        }
      }
      fence();
    }
  } else {
    epi_wave<EPI, TI, TJ>(acc, et, m0, n0 + wave * TJ * 32, g, lane);
    if constexpr (EPI == kEpiBiasGeluFp4)
      fp4_out_padding(g, m0, m0 + kNvBM, n0 / 16, (n0 + kNvBN) / 16, n0 + kNvBN >= g.N, tid, 256);
    if constexpr (EPI == kEpiFp8)
      fp8_out_padding(g, m0, m0 + kNvBM, n0 / 32, (n0 + kNvBN) / 32, n0 + kNvBN >= g.N, tid, 256);
  }
}

// The prefill schedules' conditions: NVFP4 with K % 64 == 0 (the 128 x 384
// one), MXFP8 with K % 128 == 0 (the 256 x 256 one; whole scale words), LINEAR
// scale buffers 4-byte aligned.
template <int FMT>
inline bool prefill_nv_ok(const GemmArgs& g) {
  auto word_ok = [&](const uint8_t* p, int lay) {
    return lay == kTiled || (reinterpret_cast<uintptr_t>(p) & 3) == 0;
  };
  const int64_t kmod = FMT == kMXFP8 ? 128 : 64;
  return (FMT == kNVFP4 || FMT == kMXFP8) && g.K % kmod == 0 && word_ok(g.sfa, g.la) && word_ok(g.sfb, g.lb);
}

template <int FMT, int EPI, bool SPLIT = false>
void launch_prefill_nv(const GemmArgs& g, hipStream_t s) {
  const dim3 grid((unsigned)(((g.M + kNvBM - 1) / kNvBM) * ((g.N + kNvBN - 1) / kNvBN)),
                  SPLIT ? (unsigned)g.splits : 1u),
      block(256);
  if (g.la == kTiled && g.lb == kTiled) {
    hipLaunchKernelGGL((gemm_prefill_nv_kernel<FMT, EPI, true, true, SPLIT>), grid, block, 0, s, g);
  } else if (g.la == kTiled) {
    hipLaunchKernelGGL((gemm_prefill_nv_kernel<FMT, EPI, true, false, SPLIT>), grid, block, 0, s, g);
  } else if (g.lb == kTiled) {
    hipLaunchKernelGGL((gemm_prefill_nv_kernel<FMT, EPI, false, true, SPLIT>), grid, block, 0, s, g);
  } else {
    hipLaunchKernelGGL((gemm_prefill_nv_kernel<FMT, EPI, false, false, SPLIT>), grid, block, 0, s, g);
  }
}
