// The host table builder of libtq (tq_tables.cpp) run under AddressSanitizer
// and UndefinedBehaviorSanitizer: for every config on the command line
// ("seed d bits qjl rotation", one group of five arguments each) it builds the
// tables into buffers of exactly the documented sizes (d signs twice, 2^b
// centroids, 2^b - 1 thresholds, m x d S, d x d rotation) and writes their
// bytes, in that order, to <dir>/<index>.bin, which the test compares with the
// library's exported tables.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "tq_internal.h"

namespace {

void put(std::FILE * f, const void * p, size_t n) {
    if (n && std::fwrite(p, 1, n, f) != n) std::exit(3);
}

}  // namespace

int main(int argc, char ** argv) {
    if (argc < 2 || (argc - 2) % 5 != 0) {
        std::fprintf(stderr, "usage: %s dir (seed d bits qjl rotation)...\n", argv[0]);
        return 2;
    }
    for (int a = 2, idx = 0; a + 4 < argc; a += 5, ++idx) {
        tq_config cfg;
        std::memset(&cfg, 0, sizeof cfg);
        cfg.seed = std::strtoull(argv[a], nullptr, 10);
        cfg.head_dim = std::atoi(argv[a + 1]);
        cfg.bits = std::atoi(argv[a + 2]);
        cfg.block = 32;
        cfg.qjl = std::atoi(argv[a + 3]);
        cfg.rotation = std::atoi(argv[a + 4]);
        const char * why = "";
        if (tq::validate_config(cfg, &why) != TQ_STATUS_OK) {
            std::printf("invalid %s\n", why);
            continue;
        }
        const int d = cfg.head_dim, levels = 1 << cfg.bits;
        std::vector<int8_t> d1(d), d2(d);
        std::vector<float> cb(levels), th(levels - 1), S(cfg.qjl ? size_t(d) * d : 0);
        std::vector<double> R(size_t(d) * d);
        tq::build_tables(cfg, d1.data(), d2.data(), cb.data(), th.data(), cfg.qjl ? S.data() : nullptr);
        tq::build_rotation(cfg, R.data());
        char path[4096];
        std::snprintf(path, sizeof path, "%s/%d.bin", argv[1], idx);
        std::FILE * f = std::fopen(path, "wb");
        if (!f) return 3;
        put(f, d1.data(), d1.size());
        put(f, d2.data(), d2.size());
        put(f, cb.data(), cb.size() * sizeof(float));
        put(f, th.data(), th.size() * sizeof(float));
        put(f, S.data(), S.size() * sizeof(float));
        put(f, R.data(), R.size() * sizeof(double));
        std::fclose(f);
        std::printf("ok %d\n", idx);
    }
    return 0;
}
