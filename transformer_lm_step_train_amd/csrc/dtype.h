// Activation storage types: fp32, bf16 bits (uint16_t), or IEEE fp16
// (_Float16).  Kernel launchers receive the model's type as an int.
#pragma once

enum { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };
