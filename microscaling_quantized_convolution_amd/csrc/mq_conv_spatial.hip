// mq_conv_spatial.hip -- forward and input-gradient convolutions as halo-tiled implicit GEMMs.
//
// Forward Y = W . X' and input gradient G_X = col2im(W^T . G_Y) (onedev.kr MicroQonv digest,
// section "How it differs") share one structure: an output pixel sums, over a set of taps, a
// channel contraction of one weight tap with one input pixel of a channel-batch-first tensor
// (section "How it works": per pixel all channels and batch elements are contiguous):
//
//   Out[i*sO + ah][j*sO + aw][m][n] = sum_{kh',kw'} sum_k A_tap[m][k] * In[i*SI + kh' + r0]
//                                                                        [j*SI + kw' + c0][k][n]
//   forward:            In = X,   A_tap = W[kh'][kw'],            SI = stride, r0 = -pad
//   input grad, s = 1:  In = G_Y, A_tap = W[Kh-1-kh'][Kw-1-kw']^T, r0 = pad - Kh + 1
//   input grad, s = 2:  one class per output parity (ah, aw); only the taps with
//                       kh = ah + pad (mod 2) reach it, so the class is a dense stride-1
//                       convolution with the kernel rows kh = ah + pad - 2*(r0 + kh') (no MFMA
//                       work is spent on the zeros a transposed convolution would insert).
//
// A workgroup owns 64 rows (m) x PH x PW output pixels x NB batch elements. Per 16-channel chunk
// it decodes the weight taps and the input halo ((PH-1)*SI + Kh rows x (PW-1)*SI + Kw columns)
// once into LDS as fp16 and every wave runs 32x32x16 fp16 MFMAs over all taps; the halo is read
// once per chunk and reused by every tap, and the weight tile by every pixel. The im2col matrix
// never exists outside registers. NB = 32: an MFMA's 32 columns are 32 batch elements of one
// pixel (a wave owns 64 x 4 pixels). NB = 16, for batches of at most 16: its columns are 16 batch
// elements of each of two neighbouring pixels (a wave owns 64 x 8 pixels), so a small batch
// fills the matrix core instead of padding half of every MFMA and every output store. Row
// blocks of 32 that lie wholly past the output channels (a layer with 16 or 32 of them) skip
// their MFMAs and stores.
#include "mq_kernels.hpp"
#include "mq_stage.hpp"
#include "mq_wgrad_sum.hpp"

namespace mq {

struct SpatialClass {
    int ah, aw;       // output offset of this class
    int OHs, OWs;     // class sub-grid extent
    int kh, kw;       // sub-kernel extent (0 = no tap reaches this class)
    int r0, c0;       // input offset of sub-kernel tap (0,0)
    int Ah, Bh, Aw, Bw; // weight tap row = Ah + Bh*kh', column = Aw + Bw*kw'
    int tiles_w, tiles;  // pixel tiles along the sub-grid width, total pixel tiles
    int P;               // workgroups of this class (grid row = class)
    // Set by the launch, so that a workgroup's first item and its step through the items take
    // no division on the device: tiles_h pixel tiles along the height, T items, the step P in
    // the items' mixed radix, and multipliers m with n / d = mulhi(n, m) for the divisors nblk,
    // tiles_w, tiles_h and P (exact for n * d < 2^32; m = 0 stands for d = 1).
    int tiles_h, T;
    int amax_base;       // first output-amax partial of this class's workgroups
    int step_nb, step_tj, step_ti, step_mb;
    uint32_t m_nblk, m_tw, m_th, m_P;
};

// A compile-time count passed to a generic lambda.
template <int V> struct IntC { static constexpr int value = V; };

// n / d for the multiplier m of d (see SpatialClass).
__device__ __forceinline__ int div_by(int n, uint32_t m)
{
    return m ? (int)__umulhi((uint32_t)n, m) : n;
}

struct SpatialArgs {
    const uint8_t *in_codes;
    const uint8_t *in_scales;
    const float *in_T;
    int IH, IW, K4, N4;   // input squares [IH][IW][K4][N4]
    const uint8_t *w_codes;
    const uint8_t *w_scales;
    const float *w_T;
    int Kh, Kw, Cout4, Cin4; // weight squares [Kh*Kw][Cout4][Cin4]
    float *out;
    uint32_t out_bytes;
    int OWf, M, N;        // output [..][OWf][M][N]
    int M4, nblk;         // row squares, batch blocks of 32
    int sO;
    int nclass;           // grid rows 0 .. nclass-1: convolution classes
    int sum_P;            // grid row nclass (if sum_P > 0): workgroups of the weight-gradient sum
    WgradSum sum;
    // Optional output amax (null = none): every convolution workgroup writes max |out| over the
    // outputs it wrote to amax_ws[1 + cls.amax_base + b]; workgroup 0 of class 0 writes the count
    // of partials, amax_parts, to amax_ws[0] (the tensor-amax workspace format the quantizer
    // reads with MQ_QUANTIZE_AMAX_READY).
    uint32_t *amax_ws;
    int amax_parts;
    SpatialClass cls[4];
};

// A_KR: the weight square's first dimension (Cout) is the reduction (input gradient);
// otherwise its second (Cin) is (forward). The input operand's squares always have the
// reduction (channels) along their first dimension.
//
// Waves [0, NCW) consume: MFMAs on one LDS buffer. Waves [NCW, (1+PF)*NCW) produce: they load
// the squares of the stage after next into registers and decode the next stage into the other LDS
// buffer. Both sides meet at one barrier per stage, so a SIMD runs one MFMA wave and PF decode
// waves side by side (MFMA and VALU work of different waves on one SIMD execute together).
// PF = 2 where the consumer's accumulators leave room for three waves per SIMD (32-row consumer
// waves): the decode of a 1 x 8 tile's halo and weights then keeps up with its MFMAs.
// KF = 3: every workgroup's class has the full 3 x 3 taps (compile-time tap loops, so the
// consumer's LDS reads for later taps can be issued ahead of earlier taps' MFMAs); KF = 0: the
// class's sub-kernel extent is read at run time.
// MW: 32-row blocks per consumer wave (2: a wave owns all 64 rows of 4 pixels; 1: two waves
// share 4 pixels, 32 rows each, so that small pixel tiles still give four MFMA waves).
// NB: batch elements per item (32, or 16 with two pixels per MFMA; see above).
template <int FMT, bool A_KR, int SI, int PH, int PW, int MW, int NB, int PF, int KF, bool PERSIST>
__global__ void __launch_bounds__(64 * (PH * PW / (NB == 32 ? 4 : 8)) * (2 / MW) * (1 + PF))
conv_spatial_kernel(SpatialArgs a)
{
    warm_kernel_args<SpatialArgs>();
    static_assert(NB == 32 || NB == 16, "batch block of 32 or 16");
    constexpr int PPW = NB == 32 ? 4 : 8;      // output pixels per consumer wave
    constexpr int NCW = PH * PW / PPW * (2 / MW); // consumer waves (PPW pixels x 32*MW rows each)
    constexpr int NCT = 64 * NCW;               // consumer threads
    constexpr int NP = NCT * PF;                // producer threads
    constexpr int THREADS_OF = NCT + NP;
    constexpr int KHM = 3, KWM = 3;
    constexpr int HRM = (PH - 1) * SI + KHM, HCM = (PW - 1) * SI + KWM;
    // halo columns whose operands one wave reads per kernel row: the MFMA over pixels (j, j + 1)
    // of an NB = 16 wave reads column 2j*SI + tw in its lanes 0-15 and that plus SI in 16-31
    constexpr int WCOLS = (NB == 32 ? 3 : 6) * SI + KWM;
    constexpr int HPI = NB / 4; // halo items per pixel: 4 channel squares x NB / 16 batch groups
    constexpr int ABYTES = KHM * KWM * 64 * 32, BBYTES = HRM * HCM * NB * 32;
    // producer register stages: a chunk's loads are issued RS chunk steps before its decode
    // (three or four stages measured no faster on any layer here)
    constexpr int RS = 2;
    // items: weight (tap, m4) in [0, nA), halo (pixel, n4) in [nA64, nA64 + nB); nA64 rounds nA
    // up to whole waves so that no wave runs both item kinds in one slot
    constexpr int ITEMS = ((KHM * KWM * 16 + 63) / 64 * 64 + HRM * HCM * HPI + NP - 1) / NP;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][ABYTES + BBYTES];

    // Grid (workgroups of the largest class, classes): workgroup (b, z) is number b of class z,
    // and numbers past the class's own count leave at once (a whole workgroup, before any
    // barrier). The class comes from the grid rather than a search of the classes' ranges in
    // the arguments, which put dependent argument loads before the first memory access.
    if ((int)blockIdx.y >= a.nclass) {
        // the weight gradient's split sum, riding along: one sum block per 256 lanes and
        // pass, workgroup b taking passes b, b + sum_P, ... (the loop count is the same for
        // every lane: each call below holds a barrier)
        constexpr int SG = THREADS_OF / 256;
        static_assert(THREADS_OF % 256 == 0, "the sum role takes whole 256-lane groups");
        if ((int)blockIdx.x >= a.sum_P) return;
        float4(*red)[17] = reinterpret_cast<float4(*)[17]>(lds[0]);
        const int64_t nb = wgrad_sum_blocks(a.sum);
        const int grp = (int)threadIdx.x >> 8;
        for (int64_t base = SG * (int64_t)blockIdx.x; base < nb; base += SG * (int64_t)a.sum_P) {
            wgrad_sum_block(a.sum, base + grp, (int)threadIdx.x & 255, red + 16 * grp);
            __syncthreads(); // the next pass reuses red
        }
        return;
    }
    const SpatialClass &cl = a.cls[blockIdx.y];
    if ((int)blockIdx.x >= cl.P) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_uniform(tid >> 6);
    // Work items of this class: (M block of 64 rows, pixel tile, batch block), batch block
    // fastest. Workgroup b of the class's P takes items b, b + P, ...; its chunks form one
    // stream (item-major), so the producer runs into the next item while the consumers write
    // the current one's output.
    const int tiles_h = cl.tiles_h;
    const int T = cl.T;
    const int b = xcd_number((int)blockIdx.x, cl.P);
    // PERSIST: each workgroup loops over several items; otherwise one item per workgroup
    const int nmine = b < T ? (PERSIST ? div_by(T - 1 - b, cl.m_P) + 1 : 1) : 0;
    // Item w = ((mb * tiles_h + ti) * tiles_w + tj) * nblk + nb, stepped by P in that mixed radix
    // with carries (no division per item).
    struct ItemPos { int nb, tj, ti, mb; };
    const ItemPos step_p = {cl.step_nb, cl.step_tj, cl.step_ti, cl.step_mb};
    ItemPos first;
    {
        const int q0 = div_by(b, cl.m_nblk), q1 = div_by(q0, cl.m_tw), q2 = div_by(q1, cl.m_th);
        first.nb = b - q0 * a.nblk;
        first.tj = q0 - q1 * cl.tiles_w;
        first.ti = q1 - q2 * tiles_h;
        first.mb = q2;
    }
    // The arguments the producer needs before its first load, read here, together: left to
    // the compiler, each was loaded next to its first use, and the chain of dependent
    // argument reads delayed the first load by about 0.2 us more.
    asm volatile("" ::"s"(step_p.nb), "s"(step_p.tj), "s"(step_p.ti), "s"(step_p.mb),
                 "s"(first.nb), "s"(first.tj), "s"(first.ti), "s"(first.mb), "s"(nmine));
    asm volatile("" ::"s"(cl.r0), "s"(cl.c0), "s"(cl.Ah), "s"(cl.Bh), "s"(cl.Aw), "s"(cl.Bw),
                 "s"(a.IH), "s"(a.IW), "s"(a.K4), "s"(a.N4), "s"(a.Kw), "s"(a.Cout4), "s"(a.Cin4),
                 "s"(a.M4));
    auto advance = [&](ItemPos p) {
        p.nb += step_p.nb;
        int c = p.nb >= a.nblk;
        p.nb -= c ? a.nblk : 0;
        p.tj += step_p.tj + c;
        c = p.tj >= cl.tiles_w;
        p.tj -= c ? cl.tiles_w : 0;
        p.ti += step_p.ti + c;
        c = p.ti >= tiles_h;
        p.ti -= c ? tiles_h : 0;
        p.mb += step_p.mb + c;
        return p;
    };
    const int kh = KF ? KF : cl.kh, kw = KF ? KF : cl.kw;
    const int ntap = kh * kw;
    const int HR = (PH - 1) * SI + kh, HC = (PW - 1) * SI + kw;
    const int nchunk = ((a.K4 + 3) / 4) * (ntap > 0 ? 1 : 0);
    const int G = nmine * nchunk; // chunk steps of this workgroup

    if (wave >= NCW) {
        // ================= producer =================
        const int ptid = tid - NCT;
        const int nA = ntap * 16, nA64 = (nA + 63) & ~63, nAB = nA64 + HR * HC * HPI;
        constexpr int CB = (FMT == kFP4) ? 8 : 12;
        const uint32_t in_sq = (uint32_t)a.IH * a.IW * a.K4 * a.N4;
        const uint32_t w_sq = (uint32_t)a.Kh * a.Kw * a.Cout4 * a.Cin4;
        const rsrc_t in_c = make_rsrc(a.in_codes, in_sq * CB), in_s = make_scale_rsrc(a.in_scales, in_sq);
        const rsrc_t w_c = make_rsrc(a.w_codes, w_sq * CB), w_s = make_scale_rsrc(a.w_scales, w_sq);

        // Items (all load four squares that are adjacent in memory):
        //   weight, forward: (tap, m4), squares kc0..kc0+3 of Cin, stored as four LDS rows
        //   weight, input gradient: (tap, kcl, m-group), squares 4g..4g+3 of Cin at Cout square
        //       kc0+kcl, stored as 16 LDS rows x 4 reduction elements
        //   halo: (pixel, kcl, n-group), squares 4g..4g+3 of N at channel square kc0+kcl
        // per slot, the parts that do not depend on the work item: weight square base and row
        // offset within the M block, or halo row/column and batch offset; the reduction block;
        // whether the slot holds an item at all; the LDS row
        int base0[ITEMS], off1[ITEMS], hrow[ITEMS], hcol[ITEMS], kcl_of[ITEMS], row[ITEMS];
        bool used[ITEMS];
#pragma unroll
        for (int q = 0; q < ITEMS; ++q) {
            const int it = ptid + q * NP;
            const int wit = wave_uniform(it & ~63);
            base0[q] = 0; off1[q] = 0; hrow[q] = 0; hcol[q] = 0; kcl_of[q] = 0; row[q] = 0;
            used[q] = false;
            if (wit < nA64) {
                const int t = it >> 4;
                const int tkh = t / kw, tkw = t - tkh * kw;
                const int wtap = (cl.Ah + cl.Bh * tkh) * a.Kw + (cl.Aw + cl.Bw * tkw);
                used[q] = it < nA;
                if (A_KR) {
                    const int mg = it & 3, kcl = (it >> 2) & 3;
                    base0[q] = (wtap * a.Cout4 + kcl) * a.Cin4 + 4 * mg;
                    off1[q] = 4 * mg;
                    kcl_of[q] = kcl;
                    row[q] = t * 64 + 16 * mg;
                } else {
                    base0[q] = (wtap * a.Cout4 + (it & 15)) * a.Cin4;
                    off1[q] = it & 15;
                    row[q] = t * 64 + 4 * (it & 15);
                }
            } else if (wit < nAB) {
                const int j = it - nA64, hp = j / HPI;
                const int g = NB == 32 ? (j & 1) : 0, kcl = NB == 32 ? ((j >> 1) & 3) : (j & 3);
                hrow[q] = hp / HC;
                hcol[q] = hp - hrow[q] * HC;
                off1[q] = 4 * g;
                kcl_of[q] = kcl;
                used[q] = it < nAB;
                row[q] = hp * NB + 16 * g;
            }
        }
        // RS register stages: chunk c + RS of the stream is loaded into the slot chunk c was
        // just decoded from, so every load has RS stage times to arrive. Loads are issued
        // without branches, the same number per stage (a chunk past the end loads nothing:
        // mask 0), and the loop is unrolled by RS so that slots are never copied: the
        // compiler's wait before a decode then covers exactly that chunk's loads.
        RawItem<FMT> raw[RS][ITEMS];
        // Per slot: first square of an item's chunk 0 and its static validity, for the item
        // `p`. With one item per workgroup it is set once; in the persistent case it is
        // recomputed for every load (without a branch: a branch here makes the compiler wait for
        // every load in flight).
        auto geometry = [&](ItemPos p, uint32_t (&sqb)[ITEMS], uint32_t (&vm)[ITEMS]) {
            const int nb = p.nb, m4_0 = p.mb * 16;
            const int ih0 = p.ti * PH * SI + cl.r0, iw0 = p.tj * PW * SI + cl.c0;
#pragma unroll
            for (int q = 0; q < ITEMS; ++q) {
                const bool isA = wave_uniform((ptid + q * NP) & ~63) < nA64;
                if (isA && !A_KR) {
                    sqb[q] = (uint32_t)base0[q] + (uint32_t)m4_0 * a.Cin4;
                    vm[q] = (used[q] && m4_0 + off1[q] < a.M4) ? 0xFu : 0u;
                } else if (isA) {
                    const int left = a.M4 - m4_0 - off1[q];
                    sqb[q] = (uint32_t)base0[q] + (uint32_t)m4_0;
                    vm[q] = (used[q] && left > 0) ? (left >= 4 ? 0xFu : (1u << left) - 1u) : 0u;
                } else {
                    const int ih = ih0 + hrow[q], iw = iw0 + hcol[q];
                    const int n4 = nb * (NB / 4) + off1[q];
                    const bool inside = used[q] && ih >= 0 && ih < a.IH && iw >= 0 && iw < a.IW;
                    const int left = a.N4 - n4;
                    sqb[q] = (((uint32_t)ih * a.IW + iw) * a.K4 + kcl_of[q]) * a.N4 + n4;
                    vm[q] = (inside && left > 0) ? (left >= 4 ? 0xFu : (1u << left) - 1u) : 0u;
                }
            }
        };
        uint32_t sq_chunk[ITEMS], sq_base[ITEMS], vmask[ITEMS];
#pragma unroll
        for (int q = 0; q < ITEMS; ++q) {
            const bool isA = wave_uniform((ptid + q * NP) & ~63) < nA64;
            sq_chunk[q] = isA ? (A_KR ? 4u * a.Cin4 : 4u) : 4u * a.N4;
        }
        geometry(first, sq_base, vmask);
        // the item and chunk of the next load (loads go through the stream in order)
        int lp_nb = first.nb, lp_tj = first.tj, lp_ti = first.ti, lp_mb = first.mb;
        int lc = 0;
        auto plan = [&](int gs, ItemPlan(&pl)[ITEMS]) {
            const bool valid = gs < G;
            int c = gs;
            uint32_t sqb[ITEMS], vm[ITEMS];
            if constexpr (PERSIST) {
                const ItemPos cur = {lp_nb, lp_tj, lp_ti, lp_mb};
                geometry(cur, sqb, vm);
                c = lc;
                const bool wrap = lc + 1 >= nchunk;
                const ItemPos nx = advance(cur);
                lc = wrap ? 0 : lc + 1;
                lp_nb = wrap ? nx.nb : lp_nb;
                lp_tj = wrap ? nx.tj : lp_tj;
                lp_ti = wrap ? nx.ti : lp_ti;
                lp_mb = wrap ? nx.mb : lp_mb;
            } else {
#pragma unroll
                for (int q = 0; q < ITEMS; ++q) { sqb[q] = sq_base[q]; vm[q] = vmask[q]; }
            }
            const int kvalid = a.K4 - 4 * c;
            const uint32_t kmask = kvalid >= 4 ? 0xFu : (kvalid > 0 ? (1u << kvalid) - 1u : 0u);
#pragma unroll
            for (int q = 0; q < ITEMS; ++q) {
                const bool isA = wave_uniform((ptid + q * NP) & ~63) < nA64;
                const uint32_t sq0 = sqb[q] + (uint32_t)c * sq_chunk[q];
                const bool kin = 4 * c + kcl_of[q] < a.K4;
                const uint32_t m = (isA && !A_KR) ? (vm[q] & kmask) : (kin ? vm[q] : 0u);
                pl[q] = plan_item<FMT>(sq0, valid ? m : 0u);
            }
        };
        auto issue = [&](const ItemPlan(&pl)[ITEMS], RawItem<FMT>(&dst)[ITEMS]) {
#pragma unroll
            for (int q = 0; q < ITEMS; ++q) {
                const bool isA = wave_uniform((ptid + q * NP) & ~63) < nA64;
                issue_item<FMT>(dst[q], isA ? w_c : in_c, isA ? w_s : in_s, pl[q]);
            }
        };
        auto load = [&](int gs, RawItem<FMT>(&dst)[ITEMS]) {
            ItemPlan pl[ITEMS];
            plan(gs, pl);
            issue(pl, dst);
        };
        auto store = [&](int buf, const RawItem<FMT>(&src)[ITEMS]) {
#pragma unroll
            for (int q = 0; q < ITEMS; ++q) {
                const int it = ptid + q * NP;
                const int wit = wave_uniform(it & ~63);
                if (wit < nA64) {
                    if (it < nA) {
                        if (A_KR) store_item_rows<FMT, true>(src[q], lds[buf], row[q], kcl_of[q]);
                        else store_item<FMT, false>(src[q], lds[buf], row[q]);
                    }
                } else if (wit < nAB) {
                    if (it < nAB) store_item_rows<FMT, true>(src[q], lds[buf] + ABYTES, row[q], kcl_of[q]);
                }
            }
        };
        // Step c = 0 .. G: decode chunk c from slot c % RS into LDS buffer c & 1 (chunk G does
        // not exist: the last step only waits), load chunk c + RS into that slot, and meet the
        // consumers (step 0's barrier is their first; at step c >= 1 they have just finished
        // chunk c - 1). The steps run in whole groups of RS, ending with empty steps that the
        // consumers match with barriers of their own after their last item. The loop then has a single
        // way back to its head, and the prologue only loads chunks 0 .. RS - 1, so the loop head
        // sees the same loads in flight from both sides (a step group left early made the
        // compiler wait there for every load in flight).
        //
        // The loads stay in chunk order and take their offsets from a plan made before the
        // decode: scheduling fences keep the compiler from interleaving two chunks' loads or
        // computing offsets into registers whose loads are still in flight. Either made its wait
        // before a decode cover the next chunk's loads too, which emptied the pipeline.
#pragma unroll
        for (int s = 0; s < RS; ++s) {
            __builtin_amdgcn_sched_barrier(0);
            load(s, raw[s]);
        }
        __builtin_amdgcn_sched_barrier(0);
        for (int c0 = 0; c0 <= G; c0 += RS) {
#pragma unroll
            for (int s = 0; s < RS; ++s) {
                const int c = c0 + s;
                ItemPlan pl[ITEMS];
                plan(c + RS, pl);
                __builtin_amdgcn_sched_barrier(0);
                if (c < G) store(c & 1, raw[s]);
                __builtin_amdgcn_sched_barrier(0);
                issue(pl, raw[s]);
                __builtin_amdgcn_sched_barrier(0);
                __syncthreads();
            }
        }
        if (a.amax_ws) __syncthreads(); // the consumers' output-amax reduction
        return;
    }

    // ================= consumer =================
    // (the two roles take wave-uniform branches and pass the same number of barriers)
    constexpr int WM = 2 / MW;                        // waves per pixel group
    const int wm = wave % WM, wpix = wave / WM;       // row block, pixel group
    const int wr = wpix / (PW / PPW), wp = wpix % (PW / PPW); // consumer pixel row, pixel group
    const int half = lane >> 5, l32 = lane & 31;
    const int loff = lds_row_off(l32, half);
    // NB = 16: lanes 16-31 (and 48-63) take the second pixel of each MFMA's pair
    const int h16 = l32 >> 4;
    const int loff16 = lds_row_off(l32 & 15, half);
    // Epilogue of every item: scale by T_in * T_w and store fp32. Buffer stores: an element
    // outside the output gets an out-of-range offset and is dropped; the row offset of each
    // accumulator register is a wave-uniform constant passed as soffset. The stores of one item
    // drain while the MFMAs of the next run.
    const double sd = (double)*a.in_T * (double)*a.w_T;
    const bool fsafe = scale_is_float_safe(sd);
    const float sf = (float)sd;
    const rsrc_t out_r = make_rsrc(a.out, a.out_bytes);
    // max |accumulator| over this lane's outputs, as bit patterns (a NaN sorts above every
    // number): scaled once at the end, which gives max |out| exactly (rounding the product with
    // the non-negative scale is monotonic). Padded rows and batch columns hold exact zeros, so
    // only whole pixels outside the output are left out.
    uint32_t amx = 0u;
    // Deferred output blocks (persistent launches of 64-row waves and 32-batch items): of an
    // item with a next item, whose rows and batch block are whole, the wave's last DB 32 x 32
    // blocks (u = MW - 1, j = 4 - DB .. 3) are scaled into an LDS area of the wave's own and
    // written during the next item's first chunks, 16 bytes per lane, under its MFMAs, instead
    // of in the store burst that every workgroup of the launch runs at the same moment.
    constexpr int DB = (PERSIST && NB == 32 && MW == 2) ? 2 : 0;
    __shared__ __attribute__((aligned(16))) float dstage[DB ? NCW : 1][DB ? DB : 1][32 * 32];
    uint32_t dvoff[DB ? DB : 1]; // per deferred block: the byte offset of this lane's first piece
    bool dpend = false;          // deferred blocks wait to be written (wave-uniform)
    // a lane's 16-byte piece of a block: row drow + 8 * pass, batch columns dcol .. dcol + 3
    const int drow = lane >> 3, dcol = 4 * (lane & 7);
    auto flush = [&](auto bc) {
        constexpr int B = decltype(bc)::value;
#pragma unroll
        for (int pass = 0; pass < 4; ++pass) {
            const u32x4_t v = *reinterpret_cast<const u32x4_t *>(
                &dstage[wave][B][(drow + 8 * pass) * 32 + dcol]);
            __builtin_amdgcn_raw_buffer_store_b128(v, out_r, (int)dvoff[B], pass * 8 * a.N * 4,
                                                   kStoreNT);
        }
    };
    __syncthreads();
    int gc = 0; // chunk of the stream: LDS buffer gc & 1
    ItemPos cp = first;
    for (int k = 0; k < nmine; ++k, cp = advance(cp)) {
        const int nb = cp.nb, i0 = cp.ti * PH, j0 = cp.tj * PW, m4_0 = cp.mb * 16;
        f32x16_t acc[MW][4];
#pragma unroll
        for (int u = 0; u < MW; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[u][j][r] = 0.0f;
        // Row blocks of this wave that hold output channels (wave-uniform): a block wholly past
        // M runs no MFMAs. UN = row blocks computed.
        const int rows_left = a.M - 4 * m4_0 - 32 * wm * MW;
        auto chunks = [&](auto un) {
            constexpr int UN = decltype(un)::value;
            for (int c = 0; c < nchunk; ++c, ++gc) {
                if constexpr (DB > 0) {
                    // the previous item's deferred blocks, one per chunk
                    if (dpend && c == 0) flush(IntC<0>{});
                    if (dpend && c == 1) flush(IntC<1>{});
                }
                const uint8_t *As = lds[gc & 1], *Bs = lds[gc & 1] + ABYTES;
#pragma unroll
                for (int th = 0; th < KHM; ++th) {
                    if (UN > 0 && th < kh) {
                        const int hr = wr * SI + th;
                        // every column of the wave's window is read (columns past the
                        // sub-kernel's extent stay inside the LDS buffer and are never used)
                        u32x4_t bf[WCOLS];
#pragma unroll
                        for (int cc = 0; cc < WCOLS; ++cc) {
                            if constexpr (NB == 32) {
                                const int hc = wp * 4 * SI + cc;
                                bf[cc] = *reinterpret_cast<const u32x4_t *>(
                                    Bs + lds_row_off32((hr * HC + hc) * 32, loff));
                            } else if (cc % (2 * SI) < KWM) {
                                // (stride 2: columns 4j + 3 belong to no MFMA's lanes 0-15)
                                const int P = hr * HC + wp * 8 * SI + cc + h16 * SI;
                                bf[cc] = *reinterpret_cast<const u32x4_t *>(
                                    Bs + lds_row_off16(P, loff16));
                            }
                        }
#pragma unroll
                        for (int tw = 0; tw < KWM; ++tw) {
                            if (tw < kw) {
                                const int t = th * kw + tw;
                                f16x8_t av[MW];
#pragma unroll
                                for (int u = 0; u < UN; ++u)
                                    av[u] = __builtin_bit_cast(
                                        f16x8_t, *reinterpret_cast<const u32x4_t *>(
                                                     As + lds_row_off32(t * 64 + 32 * (wm * MW + u), loff)));
#pragma unroll
                                for (int j = 0; j < 4; ++j) {
                                    const f16x8_t b =
                                        __builtin_bit_cast(f16x8_t, bf[j * (PPW / 4) * SI + tw]);
#pragma unroll
                                    for (int u = 0; u < UN; ++u)
                                        acc[u][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[u], b, acc[u][j], 0, 0, 0);
                                }
                            }
                        }
                    }
                }
                __syncthreads();
            }
        };
        if constexpr (NB == 32) {
            chunks(IntC<MW>{}); // batch blocks of 32 compute every row block (one loop copy)
            if constexpr (DB > 0) {
                // deferred blocks the chunks did not take (an item of one chunk)
                if (dpend && nchunk < 1) flush(IntC<0>{});
                if (dpend && nchunk < 2) flush(IntC<1>{});
                dpend = false;
            }
        } else {
            if (rows_left > 32 * (MW - 1)) chunks(IntC<MW>{});
            else if (rows_left > 0) chunks(IntC<1>{});
            else chunks(IntC<0>{});
        }

        const int i = i0 + wr;
        const int n = NB == 32 ? nb * 32 + l32 : nb * 16 + (l32 & 15);
        const bool full_m = 4 * m4_0 + 64 <= a.M;
        // (deferred blocks: the FS/FM copy below, for whole batch blocks of 16-byte rows)
        const bool defer = DB > 0 && k + 1 < nmine && fsafe && full_m && nb * 32 + 32 <= a.N &&
                           (a.N & 3) == 0;
        // Copies of the store loop for the scale's two forms and for whether the item's 64
        // rows all lie inside M, chosen by wave-uniform branches: with one loop the compiler
        // computed both scale forms for every element (double conversions and multiply, then a
        // select) and tested every element's row, most of the epilogue's instructions.
        auto epilogue = [&](auto fs, auto fm) {
        constexpr bool FS = decltype(fs)::value != 0, FM = decltype(fm)::value != 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int jj = j0 + wp * PPW + (NB == 32 ? j : 2 * j + h16);
            const bool pix_in = i < cl.OHs && jj < cl.OWs; // per half-wave pair for NB = 16
            const bool pix_ok = pix_in && n < a.N;
            if (a.amax_ws && pix_in) {
#pragma unroll
                for (int u = 0; u < MW; ++u)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        amx = max(amx, __float_as_uint(acc[u][j][r]) & 0x7FFFFFFFu);
            }
            const int oh = i * a.sO + cl.ah, ow = jj * a.sO + cl.aw;
#pragma unroll
            for (int u = 0; u < MW; ++u) {
                const int mrow0 = 4 * m4_0 + 32 * (wm * MW + u); // wave-uniform
                if (NB == 16 && mrow0 >= a.M) continue;          // a block of padding rows
                if constexpr (DB > 0 && FS && FM) {
                    if (u == MW - 1 && j >= 4 - DB && defer) {
                        const int B = j - (4 - DB); // (a constant once the j loop unrolls)
                        float *dst = dstage[wave][B];
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            dst[(4 * half + 8 * (r >> 2) + (r & 3)) * 32 + l32] = acc[u][j][r] * sf;
                        dvoff[B] = pix_in ? ((((uint32_t)oh * a.OWf + ow) * a.M + mrow0 + drow) * a.N +
                                             nb * 32 + dcol) * 4u
                                          : kBad;
                        continue;
                    }
                }
                const int mrow = mrow0 + 4 * half;
                const uint32_t vbase =
                    pix_ok ? ((((uint32_t)oh * a.OWf + ow) * a.M + mrow) * a.N + n) * 4u : kBad;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    // stores whose eight rows all lie past M are not issued (wave-uniform)
                    if (NB == 16 && !FM && mrow0 + 8 * (r >> 2) >= a.M) continue;
                    const int dm = 8 * (r >> 2) + (r & 3);
                    const float v = FS ? acc[u][j][r] * sf : (float)((double)acc[u][j][r] * sd);
                    const uint32_t voff = (FM || mrow + dm < a.M) ? vbase : kBad;
                    // non-temporal: the output is not read again by this pass (streaming writes
                    // measured ~10% faster than cached ones for this write-bound epilogue)
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), out_r,
                                                          (int)voff, dm * a.N * 4, kStoreNT);
                }
            }
        }
        };
        if (fsafe && full_m) epilogue(IntC<1>{}, IntC<1>{});
        else if (fsafe) epilogue(IntC<1>{}, IntC<0>{});
        else epilogue(IntC<0>{}, IntC<0>{});
        if constexpr (DB > 0) dpend = defer;
    }
    // the producer's steps past chunk G, in whole groups of its register stages
    for (int c = G + 1; c % RS != 0; ++c) __syncthreads();
    if (a.amax_ws) {
        // this workgroup's partial: the waves' maxima meet in LDS (the producers pass the same
        // barrier), scaled as the outputs were
        __shared__ uint32_t amx_red[NCW];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) amx = max(amx, (uint32_t)__shfl_xor((int)amx, off, 64));
        if (lane == 0) amx_red[wave] = amx;
        __syncthreads();
        if (tid == 0) {
            uint32_t m = amx_red[0];
#pragma unroll
            for (int w = 1; w < NCW; ++w) m = max(m, amx_red[w]);
            const float am = __uint_as_float(m);
            const float sc = fsafe ? am * sf : (float)((double)am * sd);
            a.amax_ws[1 + cl.amax_base + b] = __float_as_uint(sc) & 0x7FFFFFFFu;
            if (blockIdx.y == 0 && b == 0) a.amax_ws[0] = (uint32_t)a.amax_parts;
        }
    }
}

// ---- host side -----------------------------------------------------------------------------


// Pixel tile per workgroup: 2 x 8 for stride-1 input walks, 1 x 8 for stride 2 (whose halo is
// twice as wide), so that two LDS stage buffers fit. A stride-1 walk over a small map also takes
// the 1 x 8 tile when the 2 x 8 tiles would leave many CUs idle (see launch_spatial).
template <int SI> struct TileShape;
template <> struct TileShape<1> { static constexpr int PH = 2, PW = 8, MW = 2; };
template <> struct TileShape<2> { static constexpr int PH = 1, PW = 8, MW = 1; };

static void set_tiles(SpatialClass &c, int PH, int PW)
{
    c.tiles_w = (c.OWs + PW - 1) / PW;
    c.tiles_h = (c.OHs + PH - 1) / PH;
    c.tiles = c.tiles_w * c.tiles_h;
}

// Multiplier m of divisor d >= 1: n / d = mulhi(n, m) for n * d < 2^32 (the error of
// m = floor(2^32 / d) + 1 is below n / 2^32 < 1 / d); 0 for d = 1.
static uint32_t div_multiplier(int d)
{
    return d <= 1 ? 0u : (uint32_t)((1ull << 32) / (uint64_t)d + 1ull);
}

// The item bookkeeping of a class with its workgroup count P set.
static void set_items(SpatialClass &c, int nblk, int nmb)
{
    c.T = c.tiles * nblk * nmb;
    int r = c.P;
    c.step_nb = r % nblk; r /= nblk;
    c.step_tj = r % (c.tiles_w > 0 ? c.tiles_w : 1); r /= (c.tiles_w > 0 ? c.tiles_w : 1);
    c.step_ti = r % (c.tiles_h > 0 ? c.tiles_h : 1); r /= (c.tiles_h > 0 ? c.tiles_h : 1);
    c.step_mb = r;
    c.m_nblk = div_multiplier(nblk);
    c.m_tw = div_multiplier(c.tiles_w);
    c.m_th = div_multiplier(c.tiles_h);
    c.m_P = div_multiplier(c.P);
}

bool spatial_supported(const ConvGeom &g)
{
    if (!(g.Kh <= 3 && g.Kw <= 3 && g.sh == g.sw && (g.sh == 1 || g.sh == 2) && g.ph < g.Kh &&
          g.pw < g.Kw))
        return false;
    // 32-bit byte offsets below 2^31 for every operand and output
    const uint64_t lim = 1ull << 31;
    const uint64_t xs = (uint64_t)g.H * g.W * g.Cin4 * g.N4 * 12,
                   gs = (uint64_t)g.Ho * g.Wo * g.Cout4 * g.N4 * 12,
                   ws = (uint64_t)g.Kh * g.Kw * g.Cout4 * g.Cin4 * 12,
                   ys = (uint64_t)g.Ho * g.Wo * g.Cout * g.N * 4,
                   xo = (uint64_t)g.H * g.W * g.Cin * g.N * 4;
    if (!(xs < lim && gs < lim && ws < lim && ys < lim && xo < lim)) return false;
    // the item bookkeeping's divisions by multiplier: items * divisor < 2^32 (tiles of at least
    // 1 x 8 pixels; divisors nblk, tiles along a dimension, and at most 256 workgroups)
    const uint64_t Hm = g.H > g.Ho ? g.H : g.Ho, Wm = g.W > g.Wo ? g.W : g.Wo;
    const uint64_t tw = (Wm + 7) / 8, nblk = (g.N4 + 7) / 8;
    const uint64_t nmb = ((g.Cin4 > g.Cout4 ? g.Cin4 : g.Cout4) + 15) / 16;
    uint64_t dmax = 256;
    dmax = nblk > dmax ? nblk : dmax;
    dmax = tw > dmax ? tw : dmax;
    dmax = Hm > dmax ? Hm : dmax;
    return Hm * tw * nblk * nmb * dmax < (1ull << 32);
}

template <int FMT, bool A_KR, int SI, int PH, int PW, int MW, int NB>
static hipError_t launch_spatial_tiles(SpatialArgs &a, int nclass, hipStream_t st)
{
    constexpr int PF = MW == 1 ? 2 : 1; // producer waves per consumer wave
    constexpr int THREADS = 64 * (PH * PW / (NB == 32 ? 4 : 8)) * (2 / MW) * (1 + PF);
    constexpr int SG = THREADS / 256;   // sum blocks per workgroup pass
    int items[4] = {0, 0, 0, 0}, total = 0;
    double work[4] = {0, 0, 0, 0}, total_work = 0;
    for (int c = 0; c < nclass; ++c) {
        set_tiles(a.cls[c], PH, PW);
        items[c] = a.cls[c].tiles * a.nblk * ((a.M4 + 15) / 16);
        total += items[c];
        // per item: MFMA work in taps plus the per-chunk staging (the halo is decoded whatever
        // the tap count) and the output write, about six taps' worth
        work[c] = (double)items[c] * (a.cls[c].kh * a.cls[c].kw + 6);
        total_work += work[c];
    }
    // With at least 2.5 items per CU (4 when the classes of a stride-2 input gradient share the
    // CUs: their items differ in cost): 256 persistent workgroups (one per CU, their LDS),
    // shared among the classes by their work, each looping over items of its class, so that one
    // prologue serves several items and each item's output writes overlap the next item's
    // MFMAs. With fewer items the per-chunk bookkeeping of the loop, or an uneven split among
    // classes, measured slower than the hardware's own dispatch of one workgroup per item,
    // which is used then.
    const bool persist = total >= (nclass == 1 ? 640 : 1024);
    int nwg = 0, conv_wgs = 0;
    for (int c = 0; c < nclass; ++c) {
        int P = items[c];
        if (persist) {
            P = (int)(256.0 * work[c] / total_work);
            P = P < 1 ? 1 : (P > items[c] ? items[c] : P);
        }
        a.cls[c].P = P;
        set_items(a.cls[c], a.nblk, (a.M4 + 15) / 16);
        nwg = P > nwg ? P : nwg;
        conv_wgs += P;
    }
    a.nclass = nclass;
    // output amax: one partial per convolution workgroup, at most kAmaxParts of them (launches
    // here run fewer than 1024 workgroups; a larger one takes the amax pass over the output)
    bool amax_after = false;
    uint32_t *const amax_req = a.amax_ws;
    if (a.amax_ws) {
        int base = 0;
        for (int c = 0; c < nclass; ++c) {
            a.cls[c].amax_base = base;
            base += a.cls[c].P;
        }
        a.amax_parts = base;
        if (base > kAmaxParts || base < 1) {
            amax_after = true;
            a.amax_ws = nullptr;
        }
    }
    uint32_t *const amax_ws_after = amax_after ? amax_req : nullptr;
    if (a.sum_P < 0) {
        // The weight-gradient sum: on the CUs this launch leaves idle (one workgroup per CU:
        // the LDS), or, when it fills them, on 256 workgroups after its own. A workgroup sums
        // SG sum blocks per pass, a chain of dependent loads and a barrier (about 1.5 us),
        // so the sum rides along only when its passes hide behind the convolution or cost less
        // than a kernel of their own; otherwise it runs as its own kernel, ahead.
        const int64_t pairs = (wgrad_sum_blocks(a.sum) + SG - 1) / SG;
        const int spare = 256 - conv_wgs;
        const int64_t P = spare >= 32 ? spare : 256;
        if ((pairs + P - 1) / P <= (spare >= 32 ? 8 : 2)) {
            a.sum_P = (int)(pairs < 1 ? 1 : (pairs < P ? pairs : P));
        } else {
            a.sum_P = 0;
            const hipError_t e = launch_wgrad_sum(a.sum, st);
            if (e != hipSuccess) return e;
        }
    }
    nwg = a.sum_P > nwg ? a.sum_P : nwg;
    if (nwg == 0) return amax_ws_after ? launch_amax(a.out, a.out_bytes / 4, amax_ws_after, st)
                                       : hipSuccess;
    dim3 grid((unsigned)nwg, (unsigned)(nclass + (a.sum_P > 0 ? 1 : 0)), 1);
    const bool full3 = nclass == 1 && a.cls[0].kh == 3 && a.cls[0].kw == 3;
#define MQ_SPATIAL_LAUNCH(KFV, PV)                                                              \
    hipLaunchKernelGGL((conv_spatial_kernel<FMT, A_KR, SI, PH, PW, MW, NB, PF, KFV, PV>), grid,  \
                       dim3(THREADS), 0, st, a)
    if (full3 && persist) MQ_SPATIAL_LAUNCH(3, true);
    else if (full3) MQ_SPATIAL_LAUNCH(3, false);
    else if (persist) MQ_SPATIAL_LAUNCH(0, true);
    else MQ_SPATIAL_LAUNCH(0, false);
#undef MQ_SPATIAL_LAUNCH
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || !amax_ws_after) return e;
    return launch_amax(a.out, a.out_bytes / 4, amax_ws_after, st);
}

// Work items of either tile shape: the launch runs at most 256 workgroups (one per CU, their
// LDS), so the busiest workgroup takes ceil(items / 256) items. A 1 x 8 item does half the MFMA
// work of a 2 x 8 one in about 0.6 of its time (the per-chunk overheads stay); the shape with
// the smaller modelled time (items per workgroup x time per item) is taken.
static int spatial_grid_wgs(const SpatialArgs &a, int nclass, int PH, int PW)
{
    int max_tiles = 0;
    for (int c = 0; c < nclass; ++c) {
        const SpatialClass &k = a.cls[c];
        const int t = ((k.OWs + PW - 1) / PW) * ((k.OHs + PH - 1) / PH);
        if (t > max_tiles) max_tiles = t;
    }
    return max_tiles * a.nblk * ((a.M4 + 15) / 16) * nclass;
}

// Batch blocks: 32 elements, or for a batch of at most 16 (four squares) one block of 16 with two
// pixels per MFMA (tiles twice as wide: PW = 16).
template <int FMT, bool A_KR, int SI>
static hipError_t launch_spatial(SpatialArgs &a, int nclass, hipStream_t st)
{
    if (a.N4 <= 4) {
        a.nblk = 1;
        if constexpr (SI == 1) {
            const int w2 = spatial_grid_wgs(a, nclass, 2, 16), w1 = spatial_grid_wgs(a, nclass, 1, 16);
            const double t2 = 1.0 * ((w2 + 255) / 256), t1 = 0.6 * ((w1 + 255) / 256);
            if (t1 < t2) return launch_spatial_tiles<FMT, A_KR, SI, 1, 16, 1, 16>(a, nclass, st);
            return launch_spatial_tiles<FMT, A_KR, SI, 2, 16, 2, 16>(a, nclass, st);
        }
        return launch_spatial_tiles<FMT, A_KR, SI, 1, 16, 1, 16>(a, nclass, st);
    }
    a.nblk = (a.N4 + 7) / 8;
    constexpr int PH = TileShape<SI>::PH, PW = TileShape<SI>::PW, MW = TileShape<SI>::MW;
    if constexpr (SI == 1) {
        const int w2 = spatial_grid_wgs(a, nclass, 2, 8), w1 = spatial_grid_wgs(a, nclass, 1, 8);
        const double t2 = 1.0 * ((w2 + 255) / 256), t1 = 0.6 * ((w1 + 255) / 256);
        if (t1 < t2) return launch_spatial_tiles<FMT, A_KR, SI, 1, 8, 1, 32>(a, nclass, st);
    }
    return launch_spatial_tiles<FMT, A_KR, SI, PH, PW, MW, 32>(a, nclass, st);
}

hipError_t launch_conv_fwd_spatial(const ConvGeom &g, int fmt, QOperand x, QOperand w, float *y,
                                   hipStream_t st, uint32_t *amax_ws)
{
    SpatialArgs a = {};
    a.amax_ws = amax_ws;
    a.in_codes = x.codes; a.in_scales = x.scales; a.in_T = x.tscale;
    a.IH = g.H; a.IW = g.W; a.K4 = g.Cin4; a.N4 = g.N4;
    a.w_codes = w.codes; a.w_scales = w.scales; a.w_T = w.tscale;
    a.Kh = g.Kh; a.Kw = g.Kw; a.Cout4 = g.Cout4; a.Cin4 = g.Cin4;
    a.out = y; a.OWf = g.Wo; a.M = g.Cout; a.N = g.N; a.M4 = g.Cout4;
    a.out_bytes = (uint32_t)((uint64_t)g.Ho * g.Wo * g.Cout * g.N * 4);
    a.sO = 1;
    SpatialClass &c = a.cls[0];
    c.ah = c.aw = 0; c.OHs = g.Ho; c.OWs = g.Wo; c.kh = g.Kh; c.kw = g.Kw;
    c.r0 = -g.ph; c.c0 = -g.pw; c.Ah = 0; c.Bh = 1; c.Aw = 0; c.Bw = 1;
    if (fmt == kFP4)
        return g.sh == 1 ? launch_spatial<kFP4, false, 1>(a, 1, st)
                         : launch_spatial<kFP4, false, 2>(a, 1, st);
    return g.sh == 1 ? launch_spatial<kFP6, false, 1>(a, 1, st)
                     : launch_spatial<kFP6, false, 2>(a, 1, st);
}

// Sub-kernel of one output parity class of a stride-s input gradient along one dimension:
// the kernel offsets k with (a + pad - k) divisible by s, as a dense range of input offsets.
static void dgrad_class_dim(int a, int pad, int K, int s, int &cnt, int &r0, int &A, int &B)
{
    int kfirst = -1, klast = -1;
    for (int k = 0; k < K; ++k)
        if (((a + pad - k) % s + s) % s == 0) {
            if (kfirst < 0) kfirst = k;
            klast = k;
        }
    if (kfirst < 0) { cnt = 0; r0 = 0; A = 0; B = 0; return; }
    cnt = (klast - kfirst) / s + 1;
    r0 = (a + pad - klast) / s;   // smallest input offset (dh_min)
    A = a + pad - s * r0;         // kernel row at sub-kernel index 0
    B = -s;
}

hipError_t launch_conv_dgrad_spatial(const ConvGeom &g, int fmt, QOperand w, QOperand gy,
                                     float *gx, hipStream_t st, const WgradSum *sum,
                                     uint32_t *amax_ws)
{
    SpatialArgs a = {};
    a.amax_ws = amax_ws;
    if (sum && sum->total > 0) {
        a.sum = *sum;
        a.sum_P = -1; // sized by the launch
    }
    a.in_codes = gy.codes; a.in_scales = gy.scales; a.in_T = gy.tscale;
    a.IH = g.Ho; a.IW = g.Wo; a.K4 = g.Cout4; a.N4 = g.N4;
    a.w_codes = w.codes; a.w_scales = w.scales; a.w_T = w.tscale;
    a.Kh = g.Kh; a.Kw = g.Kw; a.Cout4 = g.Cout4; a.Cin4 = g.Cin4;
    a.out = gx; a.OWf = g.W; a.M = g.Cin; a.N = g.N; a.M4 = g.Cin4;
    a.out_bytes = (uint32_t)((uint64_t)g.H * g.W * g.Cin * g.N * 4);
    const int s = g.sh;
    a.sO = s;
    int nclass = 0;
    for (int ah = 0; ah < s; ++ah)
        for (int aw = 0; aw < s; ++aw) {
            SpatialClass &c = a.cls[nclass++];
            c.ah = ah; c.aw = aw;
            c.OHs = (g.H - ah + s - 1) / s;
            c.OWs = (g.W - aw + s - 1) / s;
            if (s == 1) {
                c.kh = g.Kh; c.kw = g.Kw;
                c.r0 = g.ph - g.Kh + 1; c.c0 = g.pw - g.Kw + 1;
                c.Ah = g.Kh - 1; c.Bh = -1; c.Aw = g.Kw - 1; c.Bw = -1;
            } else {
                dgrad_class_dim(ah, g.ph, g.Kh, s, c.kh, c.r0, c.Ah, c.Bh);
                dgrad_class_dim(aw, g.pw, g.Kw, s, c.kw, c.c0, c.Aw, c.Bw);
            }
        }
    if (fmt == kFP4) return launch_spatial<kFP4, true, 1>(a, nclass, st);
    return launch_spatial<kFP6, true, 1>(a, nclass, st);
}

} // namespace mq
