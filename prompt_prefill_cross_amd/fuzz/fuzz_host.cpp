// Host-side fuzz driver for the two parsers that read untrusted files: the
// model container parser (through ppx_model_weight_bytes, which parses and
// lays the container out without touching the GPU) and the KVCP snapshot
// check (ppx_kvfile_validate, the check ppx_kv_load and ppx_kv_load_prefix
// run before they read a snapshot).  Built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (build.py build_fuzz); any
// out-of-bounds access, overflow or leak aborts with a report.
//
//   fuzz_host <container> <snapshot> <scratch file> <iterations> <seed>
//
// Every mutated input must come back with a status (a size of 0 for a bad
// container), never a crash.  The unmutated inputs must be accepted.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <iterator>
#include <random>
#include <vector>

#include "ppx.h"

namespace {

std::vector<uint8_t> read_all(const char *path) {
    std::ifstream f(path, std::ios::binary);
    return std::vector<uint8_t>(std::istreambuf_iterator<char>(f), std::istreambuf_iterator<char>());
}

bool write_all(const char *path, const std::vector<uint8_t> &b) {
    std::FILE *f = std::fopen(path, "wb");
    if (!f) return false;
    const bool ok = std::fwrite(b.data(), 1, b.size(), f) == b.size();
    return std::fclose(f) == 0 && ok;
}

const int64_t kInteresting[] = {0, 1, -1, 2, 7, 8, 15, 16, 31, 32, 33, 63, 64, 255, 256, 257, 1023, 1024,
                                4095, 4096, 65535, 65536, 1 << 20, (1 << 20) + 1, INT32_MAX, INT32_MIN,
                                (int64_t)INT32_MAX + 1, (int64_t)UINT32_MAX, INT64_MAX, INT64_MIN,
                                (int64_t)1 << 40, (int64_t)1 << 62};

struct Mutator {
    std::mt19937_64 rng;
    explicit Mutator(uint64_t seed) : rng(seed) {}
    uint64_t below(uint64_t n) { return n ? rng() % n : 0; }
    int64_t interesting() { return kInteresting[below(sizeof(kInteresting) / sizeof(kInteresting[0]))]; }

    // one random edit; `hot` is a region (header, table) favoured for field writes
    void edit(std::vector<uint8_t> &b, size_t hot_lo, size_t hot_hi) {
        switch (below(7)) {
        case 0:  // bit flip
            if (!b.empty()) b[below(b.size())] ^= (uint8_t)(1u << below(8));
            break;
        case 1:  // byte set
            if (!b.empty()) b[below(b.size())] = (uint8_t)rng();
            break;
        case 2:
        case 3: {  // 4- or 8-byte field in the hot region set to an interesting value
            const size_t w = below(2) ? 8 : 4;
            const size_t hi = std::min(hot_hi, b.size());
            if (hi > hot_lo + w) {
                const size_t off = hot_lo + below((hi - hot_lo - w) / 4 + 1) * 4;
                const int64_t v = interesting();
                std::memcpy(b.data() + off, &v, w);
            }
            break;
        }
        case 4:  // truncate
            b.resize(below(b.size() + 1));
            break;
        case 5:  // extend
            b.resize(b.size() + 1 + below(64), (uint8_t)rng());
            break;
        default: {  // a random byte run copied from elsewhere in the input
            if (b.size() > 16) {
                const size_t n = 1 + below(16), from = below(b.size() - n), to = below(b.size() - n);
                std::memmove(b.data() + to, b.data() + from, n);
            }
            break;
        }
        }
    }
};

}  // namespace

int main(int argc, char **argv) {
    if (argc != 6) {
        std::fprintf(stderr, "usage: %s container snapshot scratch iterations seed\n", argv[0]);
        return 2;
    }
    const std::vector<uint8_t> model = read_all(argv[1]);
    const std::vector<uint8_t> snap = read_all(argv[2]);
    const char *scratch = argv[3];
    const long iters = std::atol(argv[4]);
    Mutator mu(std::strtoull(argv[5], nullptr, 10));
    if (model.size() < 128 || snap.size() < 16) {
        std::fprintf(stderr, "inputs missing or too short\n");
        return 2;
    }

    // the unmutated inputs are valid
    if (ppx_model_weight_bytes(model.data(), model.size()) == 0) {
        std::fprintf(stderr, "the seed container is rejected\n");
        return 3;
    }
    int32_t hdr[3];
    std::memcpy(hdr, snap.data() + 4, 12);
    const int nl = hdr[1], kvd = hdr[2], npos = hdr[0];
    if (!write_all(scratch, snap) || ppx_kvfile_validate(scratch, nl, kvd, npos, npos, nullptr) != PPX_OK) {
        std::fprintf(stderr, "the seed snapshot is rejected\n");
        return 3;
    }

    // the container: header (128 bytes) and the per-layer tables and tensor
    // table after it are where the parser reads fields
    long accepted = 0, rejected = 0;
    const size_t table_end = std::min<size_t>(model.size(), 128 + 8 * 64 + 96 * 256);
    for (long it = 0; it < iters; ++it) {
        std::vector<uint8_t> b = model;
        const int edits = 1 + (int)mu.below(4);
        for (int e = 0; e < edits; ++e) mu.edit(b, 8, mu.below(3) ? 128 : table_end);
        const size_t len = mu.below(8) ? b.size() : mu.below(b.size() + 1);  // also a short length over the same bytes
        const size_t need = ppx_model_weight_bytes(b.empty() ? nullptr : b.data(), len);
        (need ? accepted : rejected) += 1;
    }
    std::printf("container: %ld mutated inputs, %ld accepted, %ld rejected\n", iters, accepted, rejected);

    // the snapshot: header fields, size, token section
    accepted = rejected = 0;
    for (long it = 0; it < iters; ++it) {
        std::vector<uint8_t> b = snap;
        const int edits = 1 + (int)mu.below(3);
        for (int e = 0; e < edits; ++e) mu.edit(b, 4, mu.below(2) ? 16 : b.size());
        if (!write_all(scratch, b)) return 4;
        const int args_nl = mu.below(4) ? nl : (int)mu.interesting();
        const int args_kvd = mu.below(4) ? kvd : (int)mu.interesting();
        const int args_npos = mu.below(2) ? (int)mu.below(npos + 2) : (int)mu.interesting();
        const int args_ctx = mu.below(2) ? npos : (int)mu.interesting();
        int fpos = -7;
        const int st = ppx_kvfile_validate(scratch, args_nl, args_kvd, args_npos, args_ctx, &fpos);
        (st == PPX_OK ? accepted : rejected) += 1;
        if (st > 0) return 5;  // a status is 0 or negative
    }
    std::printf("snapshot: %ld mutated inputs, %ld accepted, %ld rejected\n", iters, accepted, rejected);
    std::remove(scratch);
    return 0;
}
