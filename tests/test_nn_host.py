"""Host-side checks of the PyTorch integration (no GPU needed)."""
from collections import Counter

from microscaling_quantized_convolution_amd.nn import MQConv2d, ResNet18MQ
import workloads


def test_resnet18_body_is_the_resnet18_workload():
    model = ResNet18MQ(num_classes=10)
    got = Counter((c.in_channels, c.out_channels, c.kernel_size, c.stride, c.padding)
                  for c in model.mq_convs)
    want = Counter((l.Cin, l.Cout, l.Kh, l.stride, l.pad) for l in workloads.config5())
    assert got == want
    assert sorted(c.layer_index for c in model.mq_convs) == list(range(19))
    assert all(c.layers == 19 for c in model.mq_convs)


def test_sr_seed_schedule():
    c = MQConv2d(4, 4, 3, layer_index=5, layers=19, seed_base=1)
    assert c.sr_seed() == 6
    c.step = 3
    assert c.sr_seed() == 1 + 5 + 19 * 3
