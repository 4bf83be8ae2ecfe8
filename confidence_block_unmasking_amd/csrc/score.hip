// Scoring half of the denoise step: every masked slot's vocabulary row reduced to per-chunk
// partial results (max, sum of exp(x - max), first index at the max).
//
// What is read ([FDFO] = page "FDFO: 让 dLLM 推理从「整批等最慢」变成「谁先完成谁先走」" §工程设计一:
// the step reads the forward's logits; only masked slots are predicted and unmasked; [DiLaServe] =
// page "DiLaServe: High SLO Attainment Serving for Diffusion Language Models" §三 3.1: the
// confidence is the softmax probability, here prepared as max, sum of exp(x - max) and argmax).
//
// How (gfx950).  A streaming reduction over M masked slots x V logits, bound by HBM.  Each row is
// cut into NC chunks of 64*kVPL 16-byte vectors (the last one shorter); the cut depends on V only,
// so a slot's result never depends on the rest of the batch.  The M*NC chunks are split evenly
// over the workgroups: four per compute unit, two resident at a time, so that as one finishes the
// dispatcher starts the next on that unit (fewer for small boxes; see launch_score).  Inside a
// workgroup the waves take chunks one at a time from an LDS counter: the sequencer favours older
// waves when they compete for the memory pipe, so a fixed split per wave leaves the young ones
// finishing last, while a shared counter lets every wave of the unit finish within about one chunk
// of the others.  (Global atomics could balance across units too, but while the logits stream one
// takes microseconds to return, longer than a wave spends on a chunk.)  One wavefront reduces one
// chunk: 64 lanes issue kVPL coalesced 16-byte non-temporal loads each (1 KiB per wave
// instruction), the next chunk's loads go out before this chunk's arithmetic, each element costs
// an unpack, a share of a max3, one FMA, one v_exp and one add (sum of exp2(x*log2e - max*log2e)),
// and lanes combine through DPP.  The chunk partial stays in a lane
// register until the wave has 64 of them or runs out of chunks, then they leave in one store: a
// store between the loads of consecutive chunks would hold back every later load until it
// completed.  No MFMA: there is no contraction here.
#include "step_common.h"

namespace dllm {

// Kernel 1: score every chunk of every masked slot.
template <bool BF16, bool ALIGNED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void score_kernel(StepParams P,
                                                                                                 int win) {
    extern __shared__ int s_id[];              // [win] slot index (row*L + j) of the window's masked slots
    __shared__ int s_tmp[2][kWaves];
    __shared__ int s_next;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = uni(tid >> 6);
    const int L = P.L, S = P.rows * L, NC = P.NC;
    const int ntiles = (S + kTile - 1) / kTile;

    // 0. Masked slots are numbered in slot order (slot = row*L + j).  Count them, then list, in
    //    LDS, those whose chunks fall in this workgroup's share.  Thread tid covers slots
    //    tid*16 .. tid*16+15 of each tile of kTile slots.
    const uint32_t mb0 = mask_bits16(P.mask_in, tid * 16, S);
    // The launch values used after the scan, fetched while the mask load is in flight (left to
    // themselves they are loaded at first use, a dependent round trip in the middle of the prologue).
    {
        const int G0 = gridDim.x, NV0 = P.NV;
        const char *lg0 = P.logits;
        const int64_t rs0 = P.row_stride_b, ps0 = P.pos_stride_b;
        const float4 *pa0 = P.partials;
        asm volatile("" ::"s"(G0), "s"(NC), "s"(NV0), "s"(lg0), "s"(rs0), "s"(ps0), "s"(pa0));
    }
    int c0 = __popc(mb0);
    const int incl0 = wave_incl_scan(c0);
    if (lane == 63) s_tmp[0][wave] = incl0;
    int more_cnt = 0;                          // masked slots in tiles 1.. (several tiles only)
    for (int k = 1; k < ntiles; ++k) more_cnt += __popc(mask_bits16(P.mask_in, k * kTile + tid * 16, S));
    __syncthreads();
    int off0 = 0, tot0 = 0;                    // tile 0: masked slots before this wave, in all
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const int v = s_tmp[0][w];
        off0 += w < wave ? v : 0;
        tot0 += v;
    }
    int M = tot0;
    if (ntiles > 1) M += block_sum(more_cnt, s_tmp[1]);
    M = uni(M);
    // share of workgroup g: I/G chunks, the first I%G workgroups one more (scalar arithmetic)
    const int I = M * NC;                      // chunk t is chunk t % NC of masked slot t / NC
    const int G = gridDim.x, g = blockIdx.x;
    const int per = I / G, rem = I - per * G;
    const int t0 = g * per + min(g, rem), t1 = t0 + per + (g < rem ? 1 : 0);
    if (t0 >= t1) return;                      // uniform over the workgroup
    const int q_lo = t0 / NC, q_hi = (t1 - 1) / NC;
    // list the slots of masked numbers q_lo..q_hi; qq = masked number of the first masked slot
    // among mb's 16, which start at slot s0.  Only the slot index is stored: the row address is
    // formed later in scalar registers (the 64-bit multiplies would cost the listing wave about
    // 0.1 us per entry here).
    auto extract = [&](uint32_t mb, int qq, int s0) {
        const int c = __popc(mb);
        if (c == 0 || qq > q_hi || qq + c <= q_lo) return;
        for (; qq < q_lo; ++qq) mb &= mb - 1;
        for (; mb != 0 && qq <= q_hi; ++qq) {
            s_id[qq - q_lo] = s0 + __builtin_ctz(mb);
            mb &= mb - 1;
        }
    };
    extract(mb0, off0 + incl0 - c0, tid * 16);
    int base = tot0;
    for (int k = 1; k < ntiles && base <= q_hi; ++k) {
        const uint32_t mb = mask_bits16(P.mask_in, k * kTile + tid * 16, S);
        const int c = __popc(mb);
        const int incl = wave_incl_scan(c);
        __syncthreads();                       // the previous user of s_tmp[1] is done
        if (lane == 63) s_tmp[1][wave] = incl;
        __syncthreads();
        int off = base, tot = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const int v = s_tmp[1][w];
            off += w < wave ? v : 0;
            tot += v;
        }
        extract(mb, off + incl - c, k * kTile + tid * 16);
        base += tot;
    }
    if (tid == 0) s_next = t0 + kWaves;
    __syncthreads();

    // 1. Chunks.  Wave w starts with chunk t0 + w, then takes the next untaken one from s_next.
    //    Which wave scores a chunk never changes the chunk's result.
    int t = t0 + wave;
    if (t >= t1) return;                       // no barrier follows
    constexpr int E = Fmt<BF16>::E;
    // lane k holds the wave's k-th pending chunk partial
    float pk_m = 0.0f, pk_s = 0.0f;
    int pk_v = 0, pk_at = 0;
    int nbuf = 0;
    // first byte of slot s's logits row (s wave-uniform: scalar arithmetic)
    auto row_of = [&](int s) -> const char * {
        const int r = s / L, j = s - r * L;
        return P.logits + (int64_t)r * P.row_stride_b + (int64_t)j * P.pos_stride_b;
    };
    int q = uni(t / NC), c = t - q * NC;
    int slot = uni(s_id[q - q_lo]);
    const char *rowp = row_of(slot);
    u32x4 raw[kVPL];
    if (ALIGNED) issue(raw, rowp, c * kCH, min(kCH, P.NV - c * kCH));
    while (true) {
        int tn = 0;
        if (lane == 0) tn = atomicAdd(&s_next, 1);
        tn = uni(tn);
        const int vb = c * kCH;
        const int n = min(kCH, P.NV - vb);
        float x[kVPL][E];
        if (ALIGNED) convert<BF16>(raw, x, n);
        else load_elems<BF16>(x, rowp, vb, n, P.V);
        const int this_at = slot * NC + c;
        // the next chunk's loads go out before this chunk's math
        const bool more = tn < t1;
        int qn = q, cn = 0;
        if (more) {
            qn = uni(tn / NC);
            cn = tn - qn * NC;
            if (qn != q) {
                slot = uni(s_id[qn - q_lo]);
                rowp = row_of(slot);
            }
            if (ALIGNED) issue(raw, rowp, cn * kCH, min(kCH, P.NV - cn * kCH));
        }
        const Part pr = reduce_lanes<E>(x, vb);
        if (lane == nbuf) {
            pk_m = pr.m;
            pk_s = pr.s;
            pk_v = pr.v;
            pk_at = this_at;
        }
        if (++nbuf == 64 || !more) {
            if (lane < nbuf) P.partials[pk_at] = make_float4(pk_m, pk_s, __int_as_float(pk_v), 0.0f);
            nbuf = 0;
        }
        if (!more) break;
        q = qn;
        c = cn;
    }
}


dllm_status launch_score(const StepParams &P, int32_t dtype, hipStream_t st, hipEvent_t ev_start, hipEvent_t ev_stop) {
    const int es = dtype == DLLM_BF16 ? 2 : 4;
    const int64_t S = (int64_t)P.rows * P.L;
    const int NC = P.NC;
    // vector path: 16-byte aligned rows whose length is a whole number of 16-byte vectors
    const bool aligned = ((uintptr_t)P.logits & 15) == 0 && (P.pos_stride_b & 15) == 0 &&
                         (P.row_stride_b & 15) == 0 && (P.V % (16 / es)) == 0;
    // grid: kGroupsPerCU workgroups per compute unit, each with an even static share; two are
    // resident on a unit at a time, and as one finishes the dispatcher starts the next on that
    // unit, which evens out the units of an XCD at the end (and overlaps each workgroup's
    // prologue with its neighbour's streaming).  Small boxes, whose chunks could not reach
    // kSmallBoxChunksPerCU per unit even if every slot were masked, take two workgroups per unit
    // (both resident at once), and the smallest (kTinyBoxChunksPerCU) one: there a workgroup would
    // otherwise get only a few chunks, and each extra workgroup is one more prologue.  More
    // workgroups when the LDS window of masked slots would exceed 2048 entries (8 KiB of dynamic
    // LDS); fewer when a fully masked box has fewer chunks than that many waves.
    const int64_t cus = cu_count();
    const int64_t box_chunks = S * NC;
    int64_t grid = cus * (box_chunks < cus * kTinyBoxChunksPerCU    ? 1
                          : box_chunks < cus * kSmallBoxChunksPerCU ? 2
                                                                   : kGroupsPerCU);
    if (grid < (S + 2047) / 2048) grid = (S + 2047) / 2048;
    const int64_t most = (S * NC + kWaves - 1) / kWaves;
    if (grid > most) grid = most;
    if (grid < 1) grid = 1;
    // window: masked slots touched by one workgroup's ceil(M*NC/grid) chunks, for M <= S
    const int64_t per = (S * NC + grid - 1) / grid;
    const int win = (int)((per + NC - 1) / NC + 2);
    const size_t lds = (size_t)win * sizeof(int);
    // with events: the same launch, the events taking the kernel's own start and end times
    auto go = [&](auto kernel) {
        if (ev_start) hipExtLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), lds, st, ev_start, ev_stop, 0, P, win);
        else hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), lds, st, P, win);
    };
    if (dtype == DLLM_BF16) {
        if (aligned) go(score_kernel<true, true>);
        else go(score_kernel<true, false>);
    } else {
        if (aligned) go(score_kernel<false, true>);
        else go(score_kernel<false, false>);
    }
    return check_hip(hipGetLastError(), "dllm_step score launch");
}


}  // namespace dllm
