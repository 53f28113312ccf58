"""MI355X-native multi-scale deformable attention (MSDeformAttn) core."""
