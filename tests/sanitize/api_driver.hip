// Sanitizer driver for the host side of the C ABI (test infrastructure):
// api.hip compiled for the host only, with AddressSanitizer and
// UndefinedBehaviorSanitizer, the kernel launchers replaced by stubs.  It
// calls every entry point with invalid arguments (no device is needed to
// refuse them), the calls that get past validation (without a GPU they stop
// at the device check), and the launch planner over a sweep of shapes up to
// the documented limits, where UBSan would catch an integer overflow.
#include "../../quantized_kv_attention_amd/csrc/api.hip"

#include <stdio.h>

namespace tqkv {
hipError_t launch_store(int, const StoreArgs &, hipStream_t) { return hipSuccess; }
hipError_t launch_verify(int, bool, int, int, bool, const VerifyArgs &, hipStream_t) { return hipSuccess; }
} // namespace tqkv

#define CHECK(cond)                                                                                                    \
    do {                                                                                                               \
        if (!(cond)) {                                                                                                 \
            printf("check failed at line %d: %s\n", __LINE__, #cond);                                                \
            return 1;                                                                                                  \
        }                                                                                                              \
    } while (0)

static int entry_points()
{
    alignas(256) static uint8_t buf[4096];
    void *dev = buf; // never dereferenced: every call below stops before a launch
    tqkv_cache c{TQKV_K3V4_NC, 2, 2, 128, 100, dev};
    size_t ws = 0;
    CHECK(tqkv_verify_workspace_bytes(nullptr, 8, 16, 0, &ws) == TQKV_ERR_ARG);
    CHECK(tqkv_verify_workspace_bytes(&c, 8, 16, 0, nullptr) == TQKV_ERR_ARG);
    tqkv_cache bad = c;
    bad.preset = 9;
    CHECK(tqkv_verify(&bad, buf, 0, (int32_t *)buf, 8, 16, 1, 0, 0.f, (float *)buf, nullptr, 0, nullptr) ==
          TQKV_ERR_ARG);
    bad = c;
    bad.D = 64;
    CHECK(tqkv_store(&bad, buf, buf, (int32_t *)buf, (int32_t *)buf, 1, nullptr) == TQKV_ERR_UNSUPPORTED);
    bad = c;
    bad.base = buf + 1;
    CHECK(tqkv_store(&bad, buf, buf, (int32_t *)buf, (int32_t *)buf, 1, nullptr) == TQKV_ERR_ALIGN);
    CHECK(tqkv_store(&c, buf, buf, (int32_t *)buf, (int32_t *)buf, -1, nullptr) == TQKV_ERR_ARG);
    CHECK(tqkv_store(&c, buf, buf, (int32_t *)buf, (int32_t *)buf, 0, nullptr) == TQKV_OK);
    CHECK(tqkv_store(&c, buf + 1, buf, (int32_t *)buf, (int32_t *)buf, 1, nullptr) == TQKV_ERR_ALIGN);
    CHECK(tqkv_verify(&c, buf + 8, 0, (int32_t *)buf, 8, 16, 1, 0, 0.f, (float *)buf, nullptr, 0, nullptr) ==
          TQKV_ERR_ALIGN);
    CHECK(tqkv_verify(&c, buf, 2, (int32_t *)buf, 8, 16, 1, 0, 0.f, (float *)buf, nullptr, 0, nullptr) ==
          TQKV_ERR_ARG);
    CHECK(tqkv_verify(&c, buf, 0, (int32_t *)buf, 8, 16, 2, 0, 0.f, (float *)buf, nullptr, 0, nullptr) ==
          TQKV_ERR_ARG);
    CHECK(tqkv_verify(&c, buf, 0, (int32_t *)buf, 8, 16, 1, -1, 0.f, (float *)buf, nullptr, 0, nullptr) ==
          TQKV_ERR_ARG);
    CHECK(tqkv_verify(&c, buf, 0, (int32_t *)buf, 8, 16, 1, 0, -1.f, (float *)buf, nullptr, 0, nullptr) ==
          TQKV_ERR_ARG);
    CHECK(tqkv_verify(&c, buf, 0, (int32_t *)buf, 8, 15, 1, 0, 0.f, (float *)buf, nullptr, 0, nullptr) ==
          TQKV_ERR_UNSUPPORTED);
    CHECK(tqkv_verify(&c, buf, 0, (int32_t *)buf, 129, 16, 1, 0, 0.f, (float *)buf, nullptr, 0, nullptr) ==
          TQKV_ERR_UNSUPPORTED);
    CHECK(tqkv_verify_noalloc(nullptr, buf, 0, (int32_t *)buf, 8, 16, 1, 0, 0.f, (float *)buf, nullptr) ==
          TQKV_ERR_ARG);
    // valid host arguments: without a gfx950 device the call stops at the device check
    const int st = tqkv_verify(&c, buf, 0, (int32_t *)buf, 8, 16, 1, 0, 0.f, (float *)buf, buf, 4096, nullptr);
    CHECK(st == TQKV_OK || st == TQKV_ERR_DEVICE || st == TQKV_ERR_WORKSPACE);
    tqkv_paged_cache pc{TQKV_K8V4, 2, 128, 10, dev, (const int32_t *)buf, 2, 7};
    CHECK(tqkv_paged_store(&pc, buf, buf, (int32_t *)buf, -3, nullptr) == TQKV_ERR_ARG);
    tqkv_paged_cache pbad = pc;
    pbad.max_pages = TQKV_MAX_PAGES_PER_SEQ + 1;
    CHECK(tqkv_paged_verify(&pbad, buf, 0, (int32_t *)buf, 8, 16, 1, 0, 0.f, (float *)buf, nullptr, 0, nullptr) ==
          TQKV_ERR_UNSUPPORTED);
    pbad = pc;
    pbad.block_table = (const int32_t *)(buf + 2);
    CHECK(tqkv_paged_verify(&pbad, buf, 0, (int32_t *)buf, 8, 16, 1, 0, 0.f, (float *)buf, nullptr, 0, nullptr) ==
          TQKV_ERR_ALIGN);
    CHECK(tqkv_verify_varlen(&c, buf, 0, (int32_t *)buf, 0, (int32_t *)buf, 16, 1, 0, 0.f, (float *)buf, nullptr, 0,
                             nullptr) != TQKV_OK);
    CHECK(tqkv_cache_bytes(TQKV_K8V4, 1 << 20, 64, 128, 1 << 23) > 0);
    CHECK(tqkv_paged_cache_bytes(TQKV_K8V4, 64, 128, INT32_MAX) == 0);
    for (int s = -7; s <= 1; ++s)
        CHECK(tqkv_status_string(s) != nullptr);
    return 0;
}

// The planner over shapes up to the limits (1 .. 2^20 sequences, up to 2^23
// tokens, every row count up to TQKV_MAX_ROWS, explicit and automatic split
// counts, contiguous and paged): the work-group counts it derives must fit
// a grid dimension whenever grid_fits says so, and the workspace must match
// the partial-state layout.
static int planner()
{
    const int Bs[] = {1, 3, 64, 4096, 1 << 20};
    const int seqs[] = {1, 31, 8192, 262144, 1 << 23};
    const int rows_list[] = {1, 8, 9, 32, 33, 64, 65, 1000, TQKV_MAX_ROWS};
    const int asks[] = {0, 1, 3, 8, 1000, 5000};
    for (int B : Bs)
        for (int S : seqs)
            for (int rows : rows_list)
                for (int ask : asks)
                    for (int paged = 0; paged < 2; ++paged) {
                        View v{TQKV_K3V4_NC, B, 8, S, (void *)16, paged ? (const int32_t *)16 : nullptr,
                               (S + 15) / 16, 1 << 26};
                        const int s = plan_splits(v, ask, 256, rows);
                        CHECK(s >= 1 && s <= 1024);
                        if (!grid_fits(v, rows, s))
                            continue;
                        const long rt = row_tiles(rows);
                        const size_t want = s > 1 ? (size_t)B * 8 * rt * s * 32 * (8 + 256) : 0;
                        // workspace_for takes n_spec and Hq: rows = (Hq / Hk) * n_spec with Hk = 8
                        if (rows % 8 == 0 && rows / 8 <= TQKV_MAX_QLEN)
                            CHECK(workspace_for(v, rows / 8, 64, s) == want);
                        (void)fuse_store(8, rows);
                    }
    return 0;
}

int main()
{
    if (entry_points() != 0)
        return 2;
    if (planner() != 0)
        return 3;
    printf("api driver ok\n");
    return 0;
}
