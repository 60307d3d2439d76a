// Host-side model description of the GPT-2 training-step library: the
// configuration's validation and defaults, the parameter table (names, shapes,
// decay and init rules, offsets in the flat fp32 buffers) and the learning-rate
// schedule. Plain C++ with no GPU dependency, so that it also builds into a
// host-only program under the compilers' sanitizers.
#ifndef GPT_MI355X_HOST_MODEL_H
#define GPT_MI355X_HOST_MODEL_H

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/gpt.h"

namespace gpth {

struct TensorInfo {
    std::string name;
    int ndim;
    int64_t shape[2];
    int64_t numel;
    int decay;
    int init;        // 0 normal, 1 proj, 2 zero, 3 one
    int64_t offset;  // element offset in the flat fp32 buffers
};

enum { INIT_NORMAL = 0, INIT_PROJ = 1, INIT_ZERO = 2, INIT_ONE = 3 };

struct LayerIdx {   // table indices of one block's tensors
    int ln1_w, ln1_b, attn_w, attn_b, proj_w, proj_b, ln2_w, ln2_b, fc_w, fc_b, mp_w, mp_b;
};

struct Table {
    std::vector<TensorInfo> t;
    int wte = -1, wpe = -1, lnf_w = -1, lnf_b = -1;
    std::vector<LayerIdx> layers;
    int64_t n_total = 0, n_decay = 0;
};

int64_t align_up(int64_t x, int64_t a);
// Parameter table of a configuration (Lecture, "Связанные веса и инициализация":
// the tied wte appears once; Linear weights [out, in]). Decayed (2-D) tensors
// first, each padded to 64 elements, then the rest.
Table build_table(const gpt_config& c);
// GPT_OK, or the status and (why non-null) the reason the configuration is rejected
gpt_status validate_config(const gpt_config* c, std::string* why);
// The GPT-2 124M configuration of the Lecture with the AdamW settings of its
// "Оптимизатор, клиппинг, расписание" section
void config_defaults(gpt_config* c);
// Warmup (it + 1) / warmup, min_lr past max_steps, cosine decay in between
// (Lecture, "Оптимизатор, клиппинг, расписание")
double lr_schedule(int32_t it, int32_t warmup, int32_t max_steps, double max_lr, double min_lr);

}  // namespace gpth

#endif  // GPT_MI355X_HOST_MODEL_H
