// Drives the host-only paths of the C ABI (descriptor checks, workspace
// planning, and the argument checks every compute entry point makes before
// it enqueues anything) for a build of api.hip with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code.  The kernel launchers of the
// other sources are stand-ins that fail the test if a call ever reaches
// them: every call below must be rejected, or be host-only, before a launch.
#include "../../include/nsa_sel.h"
#include "../../nsa_selected_block_amd/csrc/internal.h"

#include <stdio.h>
#include <stdlib.h>

namespace nsa {
static hipError_t reached(const char* what)
{
    fprintf(stderr, "launcher reached: %s\n", what);
    abort();
}
hipError_t launch_index(const Params&, int32_t*, int32_t*, hipStream_t) { return reached("index"); }
hipError_t launch_index_prebuilt(const Params&, const int32_t*, const int32_t*, int, hipStream_t)
{
    return reached("prebuilt index");
}
hipError_t launch_main(const Params&, int, hipStream_t) { return reached("main"); }
hipError_t launch_merge(const Params&, int, hipStream_t) { return reached("merge"); }
hipError_t launch_dense(const Params&, int, hipStream_t) { return reached("dense"); }
int main_grid_size(int, int, int) { (void)reached("grid"); return 0; }
hipError_t launch_bwd_delta(const Params&, int, hipStream_t) { return reached("bwd delta"); }
hipError_t launch_bwd_main(const Params&, int, hipStream_t) { return reached("bwd main"); }
hipError_t launch_bwd_dq_merge(const Params&, int, hipStream_t) { return reached("bwd dq merge"); }
int bwd_grid_size(int, int, int) { (void)reached("bwd grid"); return 0; }
hipError_t launch_prep(const Params&, hipStream_t) { return reached("prep"); }
hipError_t launch_window(const Params&, int, hipStream_t) { return reached("window"); }
hipError_t launch_window_orphans(const Params&, int, hipStream_t) { return reached("window orphans"); }
hipError_t launch_sel_prep(const Params&, hipStream_t) { return reached("select prep"); }
hipError_t launch_compress(const Params&, int, hipStream_t) { return reached("compress"); }
hipError_t launch_select(const Params&, int, int32_t*, hipStream_t) { return reached("select"); }
hipError_t launch_sel_orphans(const Params&, hipStream_t) { return reached("select orphans"); }
bool select_supported(int D, int G, int bs, int ks, int stride)
{
    return ks == 32 && stride == 16 && bs == 64 && (D == 64 || D == 128) && G >= 1 && G <= 16 && !(G & (G - 1));
}
int select_cap(int64_t T, int B) { return (int)(T / 16 + B); }
int64_t select_max_tiles(int64_t T, int B, int G) { return T / (128 / G > 0 ? 128 / G : 1) + B; }
int select_tokens(int G, int topk, int init, int local) { return G > 0 && topk > 0 && init >= 0 && local >= 0 ? 256 / G : 16; }
}  // namespace nsa

static int failures = 0;
#define EXPECT(cond)                                                    \
    do {                                                                \
        if (!(cond)) {                                                  \
            fprintf(stderr, "expectation failed: %s (line %d)\n", #cond, __LINE__); \
            ++failures;                                                 \
        }                                                               \
    } while (0)

static nsa_sel_desc good()
{
    nsa_sel_desc d{};
    d.struct_size = sizeof(nsa_sel_desc);
    d.dtype = NSA_SEL_DTYPE_BF16;
    d.num_seqs = 2;
    d.num_q_heads = 32;
    d.total_tokens = 98304;
    d.num_kv_heads = 8;
    d.head_dim = 128;
    d.block_size = 64;
    d.topk = 16;
    d.scale = 0.088f;
    d.flags = 0;
    d.stage_events = nullptr;
    return d;
}

int main()
{
    // descriptors over a grid of fields, valid and not: every host-only
    // entry point must return a status and stay in bounds
    const int dts[] = {0, 1, 2, 3, 4}, hds[] = {-1, 0, 64, 96, 128, 256}, bss[] = {0, 16, 32, 64, 128};
    const int tks[] = {0, 1, 16, 64, 65}, hqs[] = {1, 8, 30, 32, 512, 1024};
    const int64_t Ts[] = {-5, 0, 1, 4095, 98304, 12288 * 64, (int64_t)1 << 40};
    int ok = 0, n = 0;
    for (int dt : dts)
        for (int hd : hds)
            for (int bs : bss)
                for (int tk : tks)
                    for (int hq : hqs)
                        for (int64_t T : Ts) {
                            nsa_sel_desc d = good();
                            d.dtype = dt; d.head_dim = hd; d.block_size = bs; d.topk = tk;
                            d.num_q_heads = hq; d.total_tokens = T;
                            const int rc = nsa_sel_validate(&d);
                            size_t b1 = 0, b2 = 0, b3 = 0, b4 = 0, b5 = 0;
                            int64_t nb = 0, ne = 0;
                            const int r1 = nsa_sel_fwd_workspace_size(&d, &b1);
                            const int r2 = nsa_sel_index_workspace_size(&d, &b2);
                            nsa_sel_bwd_workspace_size(&d, &b3);
                            nsa_sel_window_workspace_size(&d, &b4);
                            nsa_sel_select_workspace_size(&d, &b5);
                            const int r3 = nsa_sel_index_sizes(&d, &nb, &ne);
                            EXPECT(r1 == rc && r2 == rc && r3 == rc);
                            if (rc == NSA_SEL_OK) {
                                ++ok;
                                EXPECT(b1 >= b2 && nb >= 1 && ne >= 0);
                            }
                            ++n;
                        }
    // argument checks: nothing may reach a launcher
    nsa_sel_desc d = good();
    void* p = reinterpret_cast<void*>(0x2000);
    void* ws = reinterpret_cast<void*>(0x1000);
    const int32_t* ip = static_cast<const int32_t*>(p);
    EXPECT(nsa_sel_attn_fwd(&d, nullptr, p, p, ip, ip, p, (float*)p, ws, (size_t)1 << 40, nullptr) ==
           NSA_SEL_ERR_INVALID_ARG);
    EXPECT(nsa_sel_attn_fwd(&d, p, p, p, ip, ip, p, (float*)p, ws, 1024, nullptr) == NSA_SEL_ERR_WORKSPACE);
    EXPECT(nsa_sel_attn_fwd(nullptr, p, p, p, ip, ip, p, (float*)p, ws, 1024, nullptr) == NSA_SEL_ERR_INVALID_ARG);
    EXPECT(nsa_sel_attn_fwd_indexed(&d, p, p, p, ip, ip, nullptr, ip, p, (float*)p, ws, (size_t)1 << 40, nullptr) ==
           NSA_SEL_ERR_INVALID_ARG);
    EXPECT(nsa_sel_build_index(&d, ip, ip, nullptr, (int32_t*)p, ws, (size_t)1 << 40, nullptr) ==
           NSA_SEL_ERR_INVALID_ARG);
    EXPECT(nsa_sel_build_index(&d, ip, ip, (int32_t*)p, (int32_t*)p, ws, 16, nullptr) == NSA_SEL_ERR_WORKSPACE);
    EXPECT(nsa_sel_attn_bwd(&d, p, p, p, p, (float*)p, p, ip, ip, p, p, nullptr, ws, (size_t)1 << 40, nullptr) ==
           NSA_SEL_ERR_INVALID_ARG);
    EXPECT(nsa_sel_window_fwd(&d, 0, p, p, p, ip, p, (float*)p, ws, (size_t)1 << 40, nullptr) ==
           NSA_SEL_ERR_INVALID_ARG);
    EXPECT(nsa_sel_select_blocks(&d, 32, 16, 1, 2, p, p, ip, (int32_t*)p, ws, 8, nullptr) == NSA_SEL_ERR_WORKSPACE);
    EXPECT(nsa_sel_select_blocks(&d, 33, 16, 1, 2, p, p, ip, (int32_t*)p, ws, (size_t)1 << 40, nullptr) ==
           NSA_SEL_ERR_UNSUPPORTED);
    int st = 0;
    EXPECT(nsa_sel_check(nullptr, nullptr, &st) == NSA_SEL_ERR_INVALID_ARG);
    for (int s = -7; s <= 2; ++s) EXPECT(nsa_sel_status_string(s) != nullptr);
    EXPECT(nsa_sel_last_error() != nullptr);
    EXPECT(nsa_sel_version() == NSA_SEL_ABI_VERSION);
    printf("abi host driver: %d descriptors (%d valid), %d failures\n", n, ok, failures);
    return failures ? 1 : 0;
}
