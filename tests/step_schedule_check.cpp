// Host-side check of the one-launch batch-1 step's load schedule
// (decode_step_amd/csrc/qd_step_sched.h), compiled and run by
// tests/test_step_schedule.py; no GPU is touched.
//
// For a model shape and a position it walks every workgroup's block list the way
// the kernel's loader does (qd::step::n_blocks / get_block / page_block /
// dma_src, the same functions the kernel calls) over tensors placed at known
// address ranges, and checks:
//  - every active lane's 16-byte DMA source lies inside the tensor its block
//    belongs to, and every block fits the LDS ring;
//  - each weight matrix, bias and gain of a layer is loaded exactly once by the
//    workgroups that use it (the row and column partition has no gap or overlap),
//    and the lm_head's rows once;
//  - the pages of positions 0..p of each KV head are loaded by that head's
//    attention splits;
//  - the compute waves' slot cursor (which takes the blocks in the same order)
//    agrees with the loader's at the end of every phase.
// Prints "ok" and exits 0, or prints the first failure and exits 1.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <random>
#include <string>
#include <vector>

#include "qd_step_sched.h"

using namespace qd;
using namespace qd::step;

namespace {

struct Tensor {
    std::string name;
    uint64_t base, bytes;
    std::vector<uint32_t> hits;   // per 16-byte chunk: loads within one layer's pass
};

std::vector<Tensor> g_t;
uint64_t g_next = 0x100000000ull;

int add_tensor(const std::string& name, uint64_t bytes) {
    const uint64_t rounded = (bytes + 255) / 256 * 256;
    g_t.push_back(Tensor{name, g_next, bytes, std::vector<uint32_t>((bytes + 15) / 16, 0)});
    g_next += rounded + 4096;   // a gap: a read past a tensor's end hits no tensor
    return (int)g_t.size() - 1;
}
const char* ptr(int t) { return (const char*)(uintptr_t)g_t[t].base; }

int fail(const std::string& m) {
    std::printf("FAIL: %s\n", m.c_str());
    std::exit(1);
}

// the tensor holding [a, a + 16); -1 if none (tensors sit at increasing addresses)
int owner(uint64_t a) {
    int lo = 0, hi = (int)g_t.size() - 1, at = -1;
    while (lo <= hi) {
        const int mid = (lo + hi) / 2;
        if (g_t[mid].base <= a) { at = mid; lo = mid + 1; } else hi = mid - 1;
    }
    if (at < 0 || a + 16 > g_t[at].base + ((g_t[at].bytes + 15) / 16) * 16) return -1;
    return at;
}

void run_case(int L, int D, int Hq, int Hkv, int F, int V, int p, bool bias, bool qk_norm, unsigned seed) {
    g_t.clear();
    g_next = 0x100000000ull;
    qd_config c{};
    c.n_layers = L; c.hidden = D; c.n_q_heads = Hq; c.n_kv_heads = Hkv; c.head_dim = 64; c.ffn = F;
    c.vocab = V; c.page_size = 16; c.rms_eps = 1e-6f; c.rope_theta = 1e6f; c.qk_norm = qk_norm ? 1 : 0;
    c.w_dtype = QD_BF16; c.kv_dtype = QD_BF16;
    const StepPlan sp = plan_step(&c, p + 1);
    if (!sp.ok) fail("plan_step rejected the case");
    const int hd = 64, G = Hq / Hkv;
    // a paged cache with a shuffled page order, pages for positions 0..p + 16
    const int npages = (p + 1 + 16 + 15) / 16 + 3;
    std::vector<int> table(npages);
    for (int i = 0; i < npages; ++i) table[i] = i;
    std::mt19937 rng(seed);
    std::shuffle(table.begin(), table.end(), rng);
    StepArgs a{};
    a.L = L; a.D = D; a.Hq = Hq; a.Hkv = Hkv; a.hd = hd; a.G = G; a.F = F; a.V = V;
    a.qkvr = (Hq + 2 * Hkv) * hd; a.qk_norm = qk_norm; a.has_bias = bias; a.S = sp.S; a.C = sp.C;
    a.up_wa = sp.up_wa; a.up_wb = sp.up_wb; a.down_wa = sp.down_wa; a.down_wb = sp.down_wb;
    a.max_blocks = npages; a.num_pages = npages;
    a.block_table = table.data();   // read on the host here
    std::vector<std::map<std::string, int>> lt(L);
    for (int l = 0; l < L; ++l) {
        auto& m = lt[l];
        const std::string pre = "layer" + std::to_string(l) + ".";
        m["attn_norm"] = add_tensor(pre + "attn_norm", (uint64_t)D * 2);
        m["wq"] = add_tensor(pre + "wq", (uint64_t)Hq * hd * D * 2);
        m["wk"] = add_tensor(pre + "wk", (uint64_t)Hkv * hd * D * 2);
        m["wv"] = add_tensor(pre + "wv", (uint64_t)Hkv * hd * D * 2);
        if (bias) {
            m["bq"] = add_tensor(pre + "bq", (uint64_t)Hq * hd * 2);
            m["bk"] = add_tensor(pre + "bk", (uint64_t)Hkv * hd * 2);
            m["bv"] = add_tensor(pre + "bv", (uint64_t)Hkv * hd * 2);
        }
        if (qk_norm) {
            m["q_norm"] = add_tensor(pre + "q_norm", (uint64_t)hd * 2);
            m["k_norm"] = add_tensor(pre + "k_norm", (uint64_t)hd * 2);
        }
        m["wo"] = add_tensor(pre + "wo", (uint64_t)D * Hq * hd * 2);
        m["mlp_norm"] = add_tensor(pre + "mlp_norm", (uint64_t)D * 2);
        m["w_gate"] = add_tensor(pre + "w_gate", (uint64_t)F * D * 2);
        m["w_up"] = add_tensor(pre + "w_up", (uint64_t)F * D * 2);
        m["w_down"] = add_tensor(pre + "w_down", (uint64_t)D * F * 2);
        m["kc"] = add_tensor(pre + "kc", (uint64_t)npages * Hkv * 16 * hd * 2);
        m["vc"] = add_tensor(pre + "vc", (uint64_t)npages * Hkv * 16 * hd * 2);
        StepLayer& t = a.layer[l];
        t.attn_norm = ptr(m["attn_norm"]); t.wq = ptr(m["wq"]); t.wk = ptr(m["wk"]); t.wv = ptr(m["wv"]);
        t.bq = bias ? ptr(m["bq"]) : nullptr; t.bk = bias ? ptr(m["bk"]) : nullptr; t.bv = bias ? ptr(m["bv"]) : nullptr;
        t.q_norm = qk_norm ? ptr(m["q_norm"]) : nullptr; t.k_norm = qk_norm ? ptr(m["k_norm"]) : nullptr;
        t.wo = ptr(m["wo"]); t.mlp_norm = ptr(m["mlp_norm"]); t.w_gate = ptr(m["w_gate"]); t.w_up = ptr(m["w_up"]);
        t.w_down = ptr(m["w_down"]); t.kc = (void*)ptr(m["kc"]); t.vc = (void*)ptr(m["vc"]);
    }
    const int t_fn = add_tensor("final_norm", (uint64_t)D * 2);
    const int t_lm = add_tensor("lm_head", (uint64_t)V * D * 2);
    a.final_norm = ptr(t_fn);
    a.lm_head = ptr(t_lm);

    auto load_block = [&](const Blk& b, int expect_tensor, const char* what) {
        if (blk_slots(b) > (uint32_t)kRingSlots) fail(std::string(what) + ": block larger than the ring");
        const uint32_t ns = blk_slots(b);
        for (uint32_t i = 0; i < ns; ++i)
            for (uint32_t lane = 0; lane < 64; ++lane) {
                bool on;
                const char* s = dma_src(b, i, lane, &on);
                if (!on) continue;
                const uint64_t ad = (uint64_t)(uintptr_t)s;
                const int o = owner(ad);
                if (o != expect_tensor)
                    fail(std::string(what) + ": a lane reads " + (o < 0 ? std::string("outside every tensor")
                                                                       : "inside " + g_t[o].name) +
                         " instead of " + g_t[expect_tensor].name);
                g_t[o].hits[(ad - g_t[o].base) / 16] += 1;
            }
        return ns;
    };
    std::vector<int> need_pages;   // of this position: page ids of positions 0..p
    for (int t = 0; t <= p; t += 16) need_pages.push_back(table[t / 16]);

    for (int wg = 0; wg < kWgs; ++wg) {
        Sched S{};
        S.wg = wg; S.xcd = wg % kXcd; S.slot = wg / kXcd; S.p = p;
        init_rows(a, S);
        if (S.xcd < a.Hkv && S.slot < a.S) split_pages(S.slot, a.C, p, &S.pg0, &S.npg);
        if (S.npg > kMaxPages) fail("a split holds more pages than the kernel keeps");
        uint32_t ldr = 0, cmp = 0;
        for (int l = 0; l < L; ++l) {
            auto& m = lt[l];
            for (int ph = PH_QKV; ph <= PH_DOWN; ++ph) {
                const int nb = n_blocks(a, S, ph);
                for (int k = 0; k < nb; ++k) {
                    if (ph == PH_ATTN) {
                        int kk = k;
                        if (a.qk_norm && kk < 2) {
                            ldr += load_block(get_block(a, S, l, ph, kk), m[kk == 0 ? "q_norm" : "k_norm"], "qk norm gain");
                            continue;
                        }
                        if (a.qk_norm) kk -= 2;
                        const int isv = kk >= S.npg, i = isv ? kk - S.npg : kk;
                        const int pid = table[S.pg0 + i];
                        ldr += load_block(page_block(a, l, S.xcd, pid, isv), m[isv ? "vc" : "kc"], "kv page");
                    } else {
                        const Blk b = get_block(a, S, l, ph, k);
                        const int o = owner((uint64_t)(uintptr_t)b.src);
                        if (o < 0) fail("a block starts outside every tensor");
                        ldr += load_block(b, o, "block");
                    }
                }
                // the compute waves' cursor over the same phase
                if (ph == PH_QKV && S.xcd < a.Hkv) {
                    cmp += blk_slots(get_block(a, S, l, PH_QKV, 0));
                    for (int k = 0; k < qkv_nparts(a, S.slot); ++k) {
                        if (a.has_bias) cmp += blk_slots(get_block(a, S, l, PH_QKV, 1 + 2 * k));
                        cmp += blk_slots(get_block(a, S, l, PH_QKV, a.has_bias ? 2 + 2 * k : 1 + k));
                    }
                } else if (ph == PH_ATTN && S.xcd < a.Hkv && S.slot < a.S) {
                    if (a.qk_norm) cmp += 2;
                    cmp += 4 * S.npg;   // K then V pages, 2 slots each at head_dim 64
                } else if (ph == PH_O && S.xcd < a.Hkv) {
                    cmp += blk_slots(get_block(a, S, l, PH_O, 0));
                } else if (ph == PH_UP) {
                    const int nb3 = n_blocks(a, S, PH_UP);
                    for (int k = 0; k < nb3; ++k) cmp += blk_slots(get_block(a, S, l, PH_UP, k));
                } else if (ph == PH_DOWN) {
                    cmp += blk_slots(get_block(a, S, l, PH_DOWN, 0));
                }
                if (cmp != ldr) fail("compute and loader slot cursors differ at workgroup " + std::to_string(wg));
            }
        }
        const int nh = n_blocks(a, S, PH_HEAD);
        for (int k = 0; k < nh; ++k) {
            const Blk b = get_block(a, S, 0, PH_HEAD, k);
            ldr += load_block(b, k == 0 ? t_fn : t_lm, "head");
            cmp += blk_slots(b);
        }
        if (cmp != ldr) fail("compute and loader slot cursors differ in the head");
    }
    // coverage: matrices once (per their users); gains and biases per user; pages
    const int n_grp = a.Hkv * kSlotsPerXcd;   // workgroups of the q|k|v and o_proj phases
    for (int l = 0; l < L; ++l) {
        for (auto& kv : lt[l]) {
            const Tensor& t = g_t[kv.second];
            const std::string& n = kv.first;
            uint32_t want;   // loads of every chunk
            if (n == "attn_norm") want = n_grp;
            else if (n == "mlp_norm") want = kWgs;
            else if (n == "q_norm" || n == "k_norm") want = a.Hkv * a.S;
            else if (n == "kc" || n == "vc") continue;
            else want = 1;
            for (size_t i = 0; i < t.hits.size(); ++i) {
                const bool bias_chunk = n == "bq" || n == "bk" || n == "bv";
                if (bias_chunk ? t.hits[i] < 1 : t.hits[i] != want)
                    fail(t.name + ": chunk " + std::to_string(i) + " loaded " + std::to_string(t.hits[i]) +
                         " times, want " + std::to_string(want));
            }
        }
        for (const char* kvn : {"kc", "vc"}) {
            const Tensor& t = g_t[lt[l][kvn]];
            for (int pid : need_pages)
                for (int g = 0; g < a.Hkv; ++g) {
                    const uint64_t off = ((uint64_t)pid * a.Hkv + g) * 16 * hd * 2;
                    for (uint64_t c2 = off / 16; c2 < (off + 16 * hd * 2) / 16; ++c2)
                        if (t.hits[c2] != 1) fail(t.name + ": a page of a needed position not loaded once");
                }
        }
    }
    for (size_t i = 0; i < g_t[t_lm].hits.size(); ++i)
        if (g_t[t_lm].hits[i] != 1) fail("lm_head chunk loaded " + std::to_string(g_t[t_lm].hits[i]) + " times");
    std::printf("case L=%d D=%d Hq=%d Hkv=%d F=%d V=%d p=%d bias=%d qk_norm=%d: S=%d C=%d ok\n", L, D, Hq, Hkv, F, V, p,
                (int)bias, (int)qk_norm, a.S, a.C);
}

}  // namespace

int main(int argc, char** argv) {
    const bool full = argc > 1 && std::strcmp(argv[1], "full") == 0;
    // the 0.5B shape at the positions the tests and the benchmark use, and edges
    for (int p : {0, 15, 16, 17, 37, 63, 64, 300, 512, 543, 704})
        run_case(2, 896, 14, 2, 4864, 4096, p, true, false, 7u + p);
    run_case(2, 896, 14, 2, 4864, 4096, 100, false, true, 3u);
    run_case(3, 256, 8, 4, 512, 1000, 130, true, false, 5u);
    if (full) run_case(24, 896, 14, 2, 4864, 151936, 512, true, false, 11u);
    std::printf("ok\n");
    return 0;
}
